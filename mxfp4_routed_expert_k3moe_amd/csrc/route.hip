// route.hip -- sigmoid + score-correction-bias top-K router, one wavefront per token.
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): sigmoid router plus a
// score-correction bias, top-16, raw-score renormalization; colibri PR #676
// summary: 896 routed experts per layer, top-16.
//
// Selection key: fp32(fp32(sigmoid(l)) + b) with the sigmoid evaluated in double,
// so the key is the correctly rounded value of the same expression on any device
// and selections are reproducible bit for bit.  A candidate is a 64-bit code
// (order-preserving key bits << 32 | ~id), so one unsigned max picks the largest
// key and, among equal keys, the lower id.
//
// One workgroup of 4 waves per token: wave w holds experts [w*Q, (w+1)*Q) in
// registers and finds their top-K with K rounds of a 32-bit wave max on the key
// (a second reduction on the id only when keys tie); the 4*K survivors then rank
// themselves against each other in parallel.
#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

constexpr int K3MOE_MAX_K_DEV = 64;

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
    v = max(v, dpp_u32<0x142, 0xA>(v));  // row_bcast:15 into rows 1, 3
    v = max(v, dpp_u32<0x143, 0xC>(v));  // row_bcast:31 into rows 2, 3
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

// One workgroup of 4 waves per token: wave w holds experts [w*Q, (w+1)*Q) and finds
// their top-K; then every survivor counts the survivors that beat it (its rank),
// and the K best take the output slots in rank order.  The routing weights
// renormalize the selected raw sigmoids, summed in slot order in double.
template <int PL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E, int K,
                                                    double top_p, int32_t* __restrict__ idx,
                                                    float* __restrict__ w, int32_t* __restrict__ n_kept) {
    __shared__ unsigned long long cand[4 * K3MOE_MAX_K_DEV];
    __shared__ double sel_sig[K3MOE_MAX_K_DEV];
    __shared__ int sel_id[K3MOE_MAX_K_DEV];
    extern __shared__ double sig_e[];  // [E] double sigmoid of each expert's logit
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const float* l = logits + (size_t)t * E;
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
    wave_topk<PL>(code, K, lane, cand + wave * K);
    __syncthreads();  // survivors and sigmoids are in LDS

    // rank of each survivor among all 4K (codes are unique; 0 = absent)
    const int nc = 4 * K;
    if ((int)threadIdx.x < nc) {
        const unsigned long long c = cand[threadIdx.x];
        if (c != 0ull) {
            int rank = 0;
            // nc is a multiple of 4; unrolled so the LDS reads overlap instead of
            // paying one latency each
#pragma unroll 8
            for (int i = 0; i < nc; ++i) rank += cand[i] > c;
            if (rank < K) {
                const int e = (int)(~(uint32_t)(c & 0xFFFFFFFFull));
                sel_id[rank] = e;
                sel_sig[rank] = sig_e[e];
            }
        }
    }
    __syncthreads();
    if (wave != 0) return;
    double S = 0.0;  // slot order, as in the definition (reads unrolled, sum in order)
#pragma unroll 16
    for (int k = 0; k < K; ++k) S += sel_sig[k];
    const double sig = lane < K ? sel_sig[lane] : 0.0;
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
                const double sj = sel_sig[j];
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
            if ((km >> k) & 1ull) Sk += sel_sig[k];
    }
    const unsigned long long km = __ballot(kept);
    if (kept) {  // kept slots, compacted in slot order
        const int slot = __popcll(km & ((1ull << lane) - 1ull));
        idx[(size_t)t * K + slot] = sel_id[lane];
        w[(size_t)t * K + slot] = (float)(sig / Sk);
    }
    if (lane >= m && lane < K) {  // the pruned tail (lane here is the output slot)
        idx[(size_t)t * K + lane] = K3MOE_PRUNED;
        w[(size_t)t * K + lane] = 0.0f;
    }
    if (n_kept != nullptr && lane == 0) n_kept[t] = m;
}

template <int PL>
hipError_t launch_pl(const float* logits, const float* bias, int T, int E, int K, double top_p, int32_t* idx,
                     float* w, int32_t* n_kept, hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel<PL>, dim3(T), dim3(256), (size_t)E * sizeof(double), stream, logits, bias, T, E,
                       K, top_p, idx, w, n_kept);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, double top_p, int32_t* idx,
                        float* w, int32_t* n_kept, hipStream_t stream) {
    const int per_lane = ((E + 3) / 4 + 63) / 64;  // candidates per lane in each of 4 waves
    if (per_lane <= 1) return launch_pl<1>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 2) return launch_pl<2>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 4) return launch_pl<4>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 8) return launch_pl<8>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    return launch_pl<16>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
}

}  // namespace k3moe
