// route.hip -- sigmoid + score-correction-bias top-K router, one wavefront per token.
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): sigmoid router plus a
// score-correction bias, top-16, raw-score renormalization; colibri PR #676
// summary: 896 routed experts per layer, top-16.
//
// Selection key: fp32(fp32(sigmoid(l)) + b) with the sigmoid evaluated in double,
// so the key is the correctly rounded value of the same expression on any device
// and selections are reproducible bit for bit.  Each lane holds E/64 candidates
// as 64-bit codes (order-preserving key bits << 32 | ~id), so one unsigned max
// picks the largest key and, among equal keys, the lower id.  K rounds of a wave
// max pick the top-K in descending order; the owning lane retires each winner.
#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

__device__ __forceinline__ uint32_t key_order(float k) {
    uint32_t u = __float_as_uint(k);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ double sigmoid_d(float l) { return 1.0 / (1.0 + exp(-(double)l)); }

template <int PL>
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int T, int E, int K,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
    extern __shared__ unsigned long long scode[];  // [E]
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const float* l = logits + (size_t)t * E;

    // keys, staged through LDS so the double-precision sigmoid is not unrolled
    for (int e = lane; e < E; e += 64) {
        float key = (float)sigmoid_d(l[e]) + bias[e];
        if (key != key) key = -INFINITY;
        if (key == 0.0f) key = 0.0f;  // -0 ranks as +0
        scode[e] = ((unsigned long long)key_order(key) << 32) | (unsigned long long)(~(uint32_t)e);
    }
    __syncthreads();
    unsigned long long code[PL];  // 0 = absent or already taken; every live code is larger
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int e = lane + 64 * j;
        code[j] = (e < E) ? scode[e] : 0ull;
    }

    int my_sel = 0;
    for (int k = 0; k < K; ++k) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < PL; ++j) best = code[j] > best ? code[j] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            unsigned long long o = __shfl_xor(best, off, kWave);
            best = o > best ? o : best;
        }
        const int e = (int)(~(uint32_t)(best & 0xFFFFFFFFull));
        if (lane == k) my_sel = e;
        if ((e & 63) == lane) {
            const int jj = e >> 6;
#pragma unroll
            for (int j = 0; j < PL; ++j)
                if (j == jj) code[j] = 0ull;
        }
    }

    // raw-score renormalization, summed in slot order in double
    const double sig = (lane < K) ? sigmoid_d(l[my_sel]) : 0.0;
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
    hipLaunchKernelGGL(route_kernel<PL>, dim3(T), dim3(64), (size_t)E * 8, stream, logits, bias, T, E, K,
                       idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, int32_t* idx,
                        float* w, hipStream_t stream) {
    const int per_lane = (E + 63) / 64;
    if (per_lane <= 1) return launch_pl<1>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 2) return launch_pl<2>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 4) return launch_pl<4>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 8) return launch_pl<8>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 16) return launch_pl<16>(logits, bias, T, E, K, idx, w, stream);
    if (per_lane <= 32) return launch_pl<32>(logits, bias, T, E, K, idx, w, stream);
    return launch_pl<64>(logits, bias, T, E, K, idx, w, stream);
}

}  // namespace k3moe
