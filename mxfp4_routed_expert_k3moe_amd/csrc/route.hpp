// route.hpp -- the sigmoid + score-correction-bias top-K selection of one token
// by one 256-thread workgroup (the body of the router kernel in route.hip).
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): sigmoid router plus a
// score-correction bias, top-16, raw-score renormalization; colibri PR #676
// summary: 896 routed experts per layer, top-16; K3_TOPP paragraph: top-p.
//
// Selection key: fp32(fp32(sigmoid(l)) + b) with the sigmoid evaluated in double,
// so the key is the correctly rounded value of the same expression on any device
// and selections are reproducible bit for bit.  A candidate is a 64-bit code
// (order-preserving key bits << 32 | ~id), so one unsigned max picks the largest
// key and, among equal keys, the lower id.
//
// Wave w of the 4 holds experts [w*Q, (w+1)*Q) in registers.  A threshold pass
// keeps the codes whose key is at or above a bound that provably admits the top K
// (two to three dozen of 896): each wave finds the ceil(K/4)-th largest of its own
// keys with a few rounds of a wave max, and the bound is the least of the four.
// The candidates rank themselves against each other (wave 0 alone when there
// are at most 64), and wave 0 writes the result.  When more than kCandCap codes pass (flat or tied keys), each wave
// instead finds its top-K with K rounds of a 32-bit wave max on the key (a second
// reduction on the id only when keys tie) and the 4*K survivors rank themselves.
#pragma once

#include "device.hpp"
#include "k3moe.h"

namespace k3moe {
namespace route_detail {

constexpr int K3MOE_MAX_K_DEV = K3MOE_MAX_K;

__device__ __forceinline__ uint32_t key_order(float k) {
    uint32_t u = __float_as_uint(k);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ double sigmoid_d(float l) { return 1.0 / (1.0 + exp(-(double)l)); }

// Maximum of a 32-bit unsigned value over the 64 lanes, returned to every lane:
// DPP within each row of 16 (swap neighbours, swap pairs, rotate by 4, rotate by
// 8), then row 0 -> 1 and row 2 -> 3 (row_bcast15), rows 0-1 -> 2-3
// (row_bcast31); lane 63 holds the maximum.  Rows outside a broadcast's row mask
// keep their own value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    v = dpp_max_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_max_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// A candidate: order-preserving key bits (high word) and ~id (low word), so one
// unsigned comparison ranks larger keys first and, among equal keys, lower ids.
__device__ __forceinline__ unsigned long long make_code(uint32_t korder, int e) {
    return ((unsigned long long)korder << 32) | (unsigned long long)(~(uint32_t)e);
}

// Top-K of the codes a wave holds (PL per lane, 0 = absent), K rounds: each lane
// offers its best code; the wave maximum of the key words picks the winning key,
// and only when several lanes offer that key a second reduction picks the lowest
// id among them.  The winner's lane retires it.  Winner k goes to out[k].
template <int PL>
__device__ __forceinline__ void wave_topk(unsigned long long (&code)[PL], int K, int lane, unsigned long long* out) {
    unsigned long long head = 0ull;
#pragma unroll
    for (int j = 0; j < PL; ++j) head = code[j] > head ? code[j] : head;
    for (int k = 0; k < K; ++k) {
        const uint32_t hk = (uint32_t)(head >> 32);
        const uint32_t mk = wave_max_u32(hk);
        const unsigned long long tie = __ballot(hk == mk);
        uint32_t win_lo;
        int win_lane;
        if (__builtin_expect(__popcll(tie) == 1, 1)) {
            win_lane = __ffsll((long long)tie) - 1;
            win_lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)head, win_lane);
        } else {  // equal keys in several lanes: the lowest id has the largest ~id
            const uint32_t lo = (hk == mk) ? (uint32_t)head : 0u;
            win_lo = wave_max_u32(lo);
            win_lane = __ffsll((long long)__ballot(hk == mk && (uint32_t)head == win_lo)) - 1;
        }
        const unsigned long long best = ((unsigned long long)mk << 32) | win_lo;
        if (lane == 0) out[k] = (mk == 0u && win_lo == 0u) ? 0ull : best;
        if (lane == win_lane && head != 0ull) {  // retire it and find this lane's next best
            unsigned long long nh = 0ull;
#pragma unroll
            for (int j = 0; j < PL; ++j) {
                if (code[j] == head) code[j] = 0ull;
                nh = code[j] > nh ? code[j] : nh;
            }
            head = nh;
        }
    }
}

constexpr int kCandCap = 128;  // candidates the threshold pass may keep

// LDS of one token's routing; sig_e ([E] doubles) is passed separately.
struct RouteScratch {
    uint32_t tw[4];                     // per wave: the ceil(K/4)-th largest key word it holds (0: none)
    unsigned long long pool[kCandCap];  // codes at or above the threshold
    int npool;
    unsigned long long cand[4 * K3MOE_MAX_K_DEV];
    double sel_sig[K3MOE_MAX_K_DEV];  // the selection by rank
    int sel_id[K3MOE_MAX_K_DEV];
};


// Route token logits l [E] (bias [E]); wave 0 writes the slot-order result to
// idx [K], w [K] and, when given, n_kept.  Called by all 256 threads of the
// workgroup (4 waves).  top_p outside (0, 1) keeps all K.
template <int PL>
__device__ __forceinline__ void route_block(const float* __restrict__ l, const float* __restrict__ bias, int E,
                                            int K, double top_p, RouteScratch& rs, double* sig_e,
                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                            int32_t* __restrict__ n_kept) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Q = (E + 3) / 4;  // experts per wave

    float lv[PL], bv[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {  // issue every load before the first use
        const int i = lane + 64 * j, e = wave * Q + i;
        const bool ok = i < Q && e < E;
        lv[j] = ok ? l[e] : 0.f;
        bv[j] = ok ? bias[e] : 0.f;
    }
    unsigned long long code[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int i = lane + 64 * j, e = wave * Q + i;
        code[j] = 0ull;
        if (i < Q && e < E) {
            const double sd = sigmoid_d(lv[j]);
            sig_e[e] = sd;
            float key = (float)sd + bv[j];
            if (key != key) key = -INFINITY;
            if (key == 0.0f) key = 0.0f;  // -0 ranks as +0
            code[j] = make_code(key_order(key), e);
        }
    }
    // Threshold pass.  Kw = ceil(K/4).  T_w = the Kw-th largest key word of wave w's
    // codes, counting each lane once per round (a lane may hold several codes of
    // one key, so the count is a lower bound), or 0 when the wave holds fewer.  Wave
    // w has at least Kw codes with key >= T_w, so with T = min_w T_w at least 4 Kw
    // >= K codes have key >= T: the K-th largest code overall has key >= T, and so
    // has every selected code.  The pool of codes with key >= T is about 30 of 896
    // for the 16-of-896 workloads; codes are unique, so ranking the pool gives the
    // exact selection in order.
    {
        const int Kw = (K + 3) >> 2;
        uint32_t kw[PL];
        uint32_t head = 0u;
#pragma unroll
        for (int j = 0; j < PL; ++j) {
            kw[j] = (uint32_t)(code[j] >> 32);
            head = max(head, kw[j]);
        }
        uint32_t tw = 0u;
        int counted = 0;
        for (int r = 0; r < Kw; ++r) {  // every round retires at least one code
            const uint32_t m = wave_max_u32(head);
            if (m == 0u) break;  // fewer than Kw codes in this wave
            counted += __popcll(__ballot(head == m));
            if (counted >= Kw) {
                tw = m;
                break;
            }
            if (head == m) {
                head = 0u;
#pragma unroll
                for (int j = 0; j < PL; ++j) {
                    kw[j] = kw[j] == m ? 0u : kw[j];
                    head = max(head, kw[j]);
                }
            }
        }
        if (lane == 0) rs.tw[wave] = tw;
    }
    if (threadIdx.x == 0) rs.npool = 0;
    __syncthreads();  // thresholds, sigmoids, npool
    const uint32_t T = min(min(rs.tw[0], rs.tw[1]), min(rs.tw[2], rs.tw[3]));
    {
        unsigned long long bal[PL];
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < PL; ++j) {
            bal[j] = __ballot(code[j] != 0ull && (uint32_t)(code[j] >> 32) >= T);
            cnt += __popcll(bal[j]);
        }
        int base = 0;
        if (lane == 0 && cnt != 0) base = atomicAdd(&rs.npool, cnt);
        base = __builtin_amdgcn_readfirstlane(base);
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int j = 0; j < PL; ++j) {
            const int pos = base + __popcll(bal[j] & below);
            if (((bal[j] >> lane) & 1ull) && pos < kCandCap) rs.pool[pos] = code[j];
            base += __popcll(bal[j]);
        }
    }
    __syncthreads();  // the pool
    const int npool = rs.npool;  // block-uniform
    if (npool <= kCandCap) {
        // thread i ranks pool code i against the others (same-address LDS reads are
        // broadcasts; unrolled so they overlap)
        if ((int)threadIdx.x < npool) {
            const unsigned long long c = rs.pool[threadIdx.x];
            int rank = 0;
#pragma unroll 8
            for (int i = 0; i < npool; ++i) rank += rs.pool[i] > c;
            if (rank < K) {
                const int e = (int)(~(uint32_t)(c & 0xFFFFFFFFull));
                rs.sel_id[rank] = e;
                rs.sel_sig[rank] = sig_e[e];
            }
        }
        // up to 64 codes were ranked by wave 0 itself, which uses the selection next
        if (npool > 64) __syncthreads();
    } else {
        // too many codes at the threshold (flat or tied keys): K rounds of wave maxima
        wave_topk<PL>(code, K, lane, rs.cand + wave * K);
        __syncthreads();  // survivors and sigmoids are in LDS

        // rank of each survivor among all 4K (codes are unique; 0 = absent)
        const int nc = 4 * K;
        if ((int)threadIdx.x < nc) {
            const unsigned long long c = rs.cand[threadIdx.x];
            if (c != 0ull) {
                int rank = 0;
                // nc is a multiple of 4; unrolled so the LDS reads overlap instead of
                // paying one latency each
#pragma unroll 8
                for (int i = 0; i < nc; ++i) rank += rs.cand[i] > c;
                if (rank < K) {
                    const int e = (int)(~(uint32_t)(c & 0xFFFFFFFFull));
                    rs.sel_id[rank] = e;
                    rs.sel_sig[rank] = sig_e[e];
                }
            }
        }
        __syncthreads();
    }
    // wave 0 forms the weights and writes the result (when it ranked the pool alone,
    // it wrote the selection itself, and a wave's LDS accesses complete in order)
    if (wave == 0) {
        double S = 0.0;  // slot order, as in the definition (reads unrolled, sum in order)
#pragma unroll 16
        for (int k = 0; k < K; ++k) S += rs.sel_sig[k];
        const double sig = lane < K ? rs.sel_sig[lane] : 0.0;
        int m = K;
        double Sk = S;
        bool kept = lane < K;
        if (top_p > 0.0 && top_p < 1.0) {
            // top-p: this slot's place in descending-score order (ties: lower slot first),
            // then the running sum in that order until it reaches p of the total
            int pos = K;
            if (lane < K) {
                pos = 0;
                for (int j = 0; j < K; ++j) {
                    const double sj = rs.sel_sig[j];
                    pos += (sj > sig) || (sj == sig && j < lane);
                }
            }
            const double thr = top_p * S;
            double cum = 0.0;
            for (m = 0; m < K;) {
                const int src = __ffsll((long long)__ballot(pos == m)) - 1;
                cum += __longlong_as_double(((long long)(uint32_t)__builtin_amdgcn_readlane(
                                                 (int)(__double_as_longlong(sig) >> 32), src) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane((int)__double_as_longlong(sig), src));
                ++m;
                if (cum >= thr) break;
            }
            kept = pos < m;
            Sk = 0.0;  // kept scores, slot order
            const unsigned long long km = __ballot(kept);
            for (int k = 0; k < K; ++k)
                if ((km >> k) & 1ull) Sk += rs.sel_sig[k];
        }
        const unsigned long long km = __ballot(kept);
        if (kept) {  // kept slots, compacted in slot order
            const int slot = __popcll(km & ((1ull << lane) - 1ull));
            idx[slot] = rs.sel_id[lane];
            w[slot] = (float)(sig / Sk);
        }
        if (lane >= m && lane < K) {  // the pruned tail (lane here is the output slot)
            idx[lane] = K3MOE_PRUNED;
            w[lane] = 0.0f;
        }
        if (lane == 0 && n_kept != nullptr) *n_kept = m;
    }
}

// Candidates per lane in each of the 4 waves for E experts (the PL template argument).
inline int route_per_lane(int E) { return ((E + 3) / 4 + 63) / 64; }

}  // namespace route_detail
}  // namespace k3moe
