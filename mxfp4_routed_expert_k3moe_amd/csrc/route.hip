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
// registers and finds their top-K with K rounds of a wave max (the owning lane
// retires each winner); wave 0 then merges the 4*K survivors the same way and
// renormalizes the selected raw scores.
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

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((unsigned long long)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ unsigned long long dpp_keep_u64(unsigned long long v) {
    // rows outside ROW_MASK keep their own value
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF,
                                               false);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Maximum over the 64 lanes, returned to every lane: DPP within each row of 16
// (swap neighbours, swap pairs, rotate by 4, rotate by 8), then row 0 -> 1 and
// row 2 -> 3 (row_bcast15), rows 0-1 -> 2-3 (row_bcast31); lane 63 holds the
// maximum, which readlane hands to the whole wave.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max_u64(v, dpp_u64<0x124>(v));  // row_ror:4
    v = max_u64(v, dpp_u64<0x128>(v));  // row_ror:8
    v = max_u64(v, dpp_keep_u64<0x142, 0xA>(v));  // row_bcast:15 into rows 1, 3
    v = max_u64(v, dpp_keep_u64<0x143, 0xC>(v));  // row_bcast:31 into rows 2, 3
    return readlane_u64(v, 63);
}

// K rounds of a wave max over per-lane code arrays; lane k keeps winner k in
// `mine` and, if `out` is given, lane 0 also writes it to out[k].  Codes equal to
// 0 are absent (a round that finds none yields 0).
template <int PL>
__device__ __forceinline__ void wave_topk(unsigned long long (&code)[PL], int K, int lane,
                                          unsigned long long* out, unsigned long long& mine) {
    for (int k = 0; k < K; ++k) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < PL; ++j) best = code[j] > best ? code[j] : best;
        best = wave_max_u64(best);
        if (out != nullptr && lane == 0) out[k] = best;
        if (lane == k) mine = best;
        if (best != 0ull) {
#pragma unroll
            for (int j = 0; j < PL; ++j)
                if (code[j] == best) code[j] = 0ull;  // codes are unique (they carry the id)
        }
    }
}

template <int PL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E, int K,
                                                    int32_t* __restrict__ idx, float* __restrict__ w) {
    __shared__ unsigned long long cand[4 * K3MOE_MAX_K_DEV];
    extern __shared__ double sig_e[];  // [E] double sigmoid of each expert's logit
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const float* l = logits + (size_t)t * E;
    const int Q = (E + 3) / 4;  // experts per wave

    unsigned long long code[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int i = lane + 64 * j;
        const int e = wave * Q + i;
        code[j] = 0ull;
        if (i < Q && e < E) {
            const double sd = sigmoid_d(l[e]);
            sig_e[e] = sd;
            float key = (float)sd + bias[e];
            if (key != key) key = -INFINITY;
            if (key == 0.0f) key = 0.0f;  // -0 ranks as +0
            code[j] = ((unsigned long long)key_order(key) << 32) | (unsigned long long)(~(uint32_t)e);
        }
    }
    unsigned long long mine = 0ull;
    wave_topk<PL>(code, K, lane, cand + wave * K, mine);
    __syncthreads();  // the only barrier: survivors and sigmoids are in LDS
    if (wave != 0) return;

    unsigned long long mc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = lane + 64 * j;
        mc[j] = (i < 4 * K) ? cand[i] : 0ull;
    }
    wave_topk<4>(mc, K, lane, nullptr, mine);
    const int my_sel = (lane < K) ? (int)(~(uint32_t)(mine & 0xFFFFFFFFull)) : 0;

    // raw-score renormalization, summed in slot order in double
    const double sig = (lane < K) ? sig_e[my_sel] : 0.0;
    double denom = 0.0;
    for (int k = 0; k < K; ++k) denom += __shfl(sig, k, kWave);
    if (lane < K) {
        idx[(size_t)t * K + lane] = my_sel;
        w[(size_t)t * K + lane] = (float)(sig / denom);
    }
}

template <int PL>
hipError_t launch_pl(const float* logits, const float* bias, int T, int E, int K, int32_t* idx,
                     float* w, hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel<PL>, dim3(T), dim3(256), (size_t)E * sizeof(double), stream, logits, bias, T, E,
                       K, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, int32_t* idx,
                        float* w, hipStream_t stream) {
    const int per_lane = ((E + 3) / 4 + 63) / 64;  // candidates per lane in each of 4 waves
    if (per_lane <= 1) return launch_pl<1>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 2) return launch_pl<2>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 4) return launch_pl<4>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 8) return launch_pl<8>(logits, bias, T, E, K, idx, w, stream);
    return launch_pl<16>(logits, bias, T, E, K, idx, w, stream);
}

}  // namespace k3moe
