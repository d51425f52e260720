// probe.hip -- measurement kernels for the achievable peaks the benchmark reports
// beside the published ones: a streaming HBM read and MFMA issue loops.  They
// compute nothing of the routed-expert block.
//
// Streaming read: every thread reads 16-byte chunks of the buffer in a grid-stride
// loop with `unroll` chunks in flight, combining them with XOR; one dword per
// workgroup is written at the end (the data must not be dead).
//
// MFMA loop: every wave issues `iters` rounds of eight independent MFMAs of one
// kind on register operands, so the matrix pipe always has a ready instruction;
// the accumulators are summed into one float per wave.
#include <type_traits>

#include "device.hpp"
#include "k3moe.h"

namespace k3moe {
namespace {

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (NT)
                v[u] = __builtin_nontemporal_load(buf + i + u * stride);
            else
                v[u] = buf[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t part[256 / kWave];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

typedef int v8i __attribute__((ext_vector_type(8)));

typedef float f32x16 __attribute__((ext_vector_type(16)));

// kind 0: v_mfma_f32_16x16x32_bf16; 1: scaled 16x16x128 FP8 (E4M3) x FP4;
// 2: scaled 16x16x128 FP4 x FP4; 3: scaled 16x16x128 FP8 x FP8;
// 4: v_mfma_f32_32x32x16_bf16; 5: scaled 32x32x64 FP4 x FP4; 6: scaled 32x32x64 FP8 x FP4.
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    constexpr bool BIG = KIND >= 4;
    using acc_t = typename std::conditional<BIG, f32x16, f32x4>::type;
    acc_t acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = acc_t{};
    // small operands (so nothing overflows), different per lane
    const uint32_t w = 0x3C003C00u + (uint32_t)lane;  // bf16 pairs near 2^-7
    const int x = (int)(w & 0x11111111u);             // small FP8 / FP4 codes
    // A and B in distinct registers (two sets each), loaded once
    bf16x8 ab[2], bb[2];
    v8i ai[2], bi[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        ab[q] = __builtin_bit_cast(bf16x8, u32x4{w, w ^ (uint32_t)q, w, w});
        bb[q] = __builtin_bit_cast(bf16x8, u32x4{w ^ 1u, w, w ^ (uint32_t)q, w});
        ai[q] = v8i{x, x ^ q, x, x, x, x, x, x};
        bi[q] = v8i{x ^ 1, x, x ^ q, x, x, x, x, x};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (KIND == 0) {
                acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[k & 1], bb[k & 1], acc[k], 0, 0, 0);
            } else if constexpr (KIND == 4) {
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[k & 1], bb[k & 1], acc[k], 0, 0, 0);
            } else if constexpr (KIND >= 5) {
                constexpr int FA = (KIND == 5) ? 4 : 0;
                acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ai[k & 1], bi[k & 1], acc[k], FA, 4, 0, 127, 0,
                                                                         127);
            } else {
                constexpr int FA = (KIND == 2) ? 4 : 0, FB = (KIND == 3) ? 0 : 4;
                acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ai[k & 1], bi[k & 1], acc[k], FA, FB, 0, 127,
                                                                          0, 127);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    s = wave_sum(s);
    if (lane == 0) out[(blockIdx.x * blockDim.x + threadIdx.x) / kWave] = s;
}

}  // namespace
}  // namespace k3moe

extern "C" {

int k3moe_probe_stream_read(const void* buf, size_t bytes, int32_t unroll, int32_t nontemporal, int32_t blocks,
                            uint32_t* sink, void* stream) {
    using namespace k3moe;
    if (!buf || !sink) return K3MOE_E_NULL;
    if (bytes < 16 || bytes % 16 || blocks < 1 || (unroll != 4 && unroll != 8 && unroll != 16))
        return K3MOE_E_DIM;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return K3MOE_E_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* b = static_cast<const u32x4*>(buf);
    const size_t n16 = bytes / 16;
#define K3_PROBE(U)                                                                                   \
    if (unroll == U) {                                                                                \
        if (nontemporal)                                                                              \
            hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(blocks), dim3(256), 0, s, b, n16, sink); \
        else                                                                                          \
            hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(blocks), dim3(256), 0, s, b, n16, sink); \
    }
    K3_PROBE(4)
    K3_PROBE(8)
    K3_PROBE(16)
#undef K3_PROBE
    return hipGetLastError() == hipSuccess ? K3MOE_OK : K3MOE_E_HIP;
}

int k3moe_probe_mfma(int32_t kind, int32_t iters, int32_t blocks, float* out, void* stream) {
    using namespace k3moe;
    if (!out) return K3MOE_E_NULL;
    if (kind < 0 || kind > 6 || iters < 1 || blocks < 1) return K3MOE_E_DIM;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        case 1: hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        case 2: hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        case 3: hipLaunchKernelGGL(mfma_loop_kernel<3>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        case 4: hipLaunchKernelGGL(mfma_loop_kernel<4>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        case 5: hipLaunchKernelGGL(mfma_loop_kernel<5>, dim3(blocks), dim3(256), 0, s, iters, out); break;
        default: hipLaunchKernelGGL(mfma_loop_kernel<6>, dim3(blocks), dim3(256), 0, s, iters, out); break;
    }
    return hipGetLastError() == hipSuccess ? K3MOE_OK : K3MOE_E_HIP;
}

}  // extern "C"
