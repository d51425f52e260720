// latent.hip -- the LatentMoE block around the routed experts.
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): latent 7168 <-> 3584
// projections around the experts, RMSNorm on the aggregate, two fused shared
// experts, SiTU-GLU; PR #676 summary: the routed experts run in the latent space
// behind shared down/up projections, plus two fused full-width shared experts.
// Per token with hidden state h [Dh] (bf16):
//   x   = Wdn h                           [Dl]   dense GEMM, bf16 out (the activation format
//                                                of the routed chunk path; widened to fp32
//                                                for the one-token decode path)
//   a   = sum_k w_k E_k(x)                [Dl]   the routed block: decode GEMVs for one
//                                                token, the grouped chunk GEMMs otherwise
//   r   = gn * a / sqrt(mean(a^2) + eps)  [Dl]   rmsnorm kernel, bf16 out
//   out = Wup r                           [Dh]   dense GEMM, fp32
//   g   = Sg h, u = Su h                  [Fs]   dense GEMMs, fp32
//   s   = SiTU(g, u)                      [Fs]   situ kernel, bf16 out
//   out += Sd s                           [Dh]   dense GEMM accumulating into out
// The five dense products are plain bf16 GEMMs with fp32 accumulation and go to
// rocBLAS (Tensile's MFMA kernels for gfx950); the routed block, the norm and
// the activation are this library's kernels.
#include <rocblas/rocblas.h>

#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// One workgroup per token row (n <= 8192, a multiple of 32): every load is issued
// up front (up to 8 float4 of the row and 4 bf16x8 of the weight per thread), the
// sum of squares is reduced in a fixed order in fp32, then r = g * a * rsqrt(mean +
// eps) is rounded to bf16 from the registers.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ a, const uint16_t* __restrict__ g,
                                                      int n, float eps, uint16_t* __restrict__ r) {
    __shared__ float part[256 / kWave];
    const float4* row = reinterpret_cast<const float4*>(a + (size_t)blockIdx.x * n);
    const int n4 = n >> 2;
    float4 v[8];
    uint2 gw[8];  // the four bf16 weights of each float4
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        const bool ok = i < n4;
        v[j] = ok ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        gw[j] = ok ? reinterpret_cast<const uint2*>(g)[i] : make_uint2(0u, 0u);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < 256 / kWave; ++j) tot += part[j];
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
    uint2* out = reinterpret_cast<uint2*>(r + (size_t)blockIdx.x * n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        if (i >= n4) break;
        const float g0 = __uint_as_float(gw[j].x << 16), g1 = __uint_as_float(gw[j].x & 0xFFFF0000u);
        const float g2 = __uint_as_float(gw[j].y << 16), g3 = __uint_as_float(gw[j].y & 0xFFFF0000u);
        out[i] = make_uint2(pack_bf16x2(g0 * (v[j].x * inv), g1 * (v[j].y * inv)),
                            pack_bf16x2(g2 * (v[j].z * inv), g3 * (v[j].w * inv)));
    }
}

// bf16 -> fp32 (exact).
__global__ __launch_bounds__(256) void widen_kernel(const uint16_t* __restrict__ x, int n, float* __restrict__ y) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        y[i] = __uint_as_float((uint32_t)x[i] << 16);
}

// s = SiTU-GLU(g, u) elementwise, bf16 out.
__global__ __launch_bounds__(256) void situ_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                   size_t n, uint16_t* __restrict__ s) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        s[i] = (uint16_t)f32_to_bf16_bits(situ_fast(g[i], u[i]));
}

int grid_blocks(size_t n, int per_block) {
    size_t b = (n + per_block - 1) / per_block;
    return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

// One rocBLAS handle per device, created on first use.
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

hipError_t blas_for(hipStream_t stream, rocblas_handle* out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) return hipErrorUnknown;
    if (rocblas_set_stream(g_blas[dev], stream) != rocblas_status_success) return hipErrorUnknown;
    *out = g_blas[dev];
    return hipSuccess;
}

// out[T, N] (fp32 or bf16, row-major) = beta * out + in[T, Kd] (bf16) . W[N, Kd]^T (bf16):
// in column-major terms out^T = W^T^T . in^T with W read transposed.
hipError_t dense(rocblas_handle h, const uint16_t* in, int T, int Kd, const uint16_t* W, int N, void* out,
                 bool out_f32, float beta) {
    const float alpha = 1.0f;
    const rocblas_datatype ot = out_f32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
    const rocblas_status st =
        rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, T, Kd, &alpha, W,
                        rocblas_datatype_bf16_r, Kd, in, rocblas_datatype_bf16_r, Kd, &beta, out, ot, N, out, ot, N,
                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace

// x (bf16, and fp32 for one token), the routed block's workspace, a, r, g, u, s.
size_t latent_workspace_bytes(const LatentDims& L, int T, int K, int E) {
    const size_t t = (size_t)T;
    const size_t routed = T == 1 ? decode_workspace_bytes(K, L.Dl, L.F) : chunk_workspace_bytes(T, K, E, L.Dl, L.F);
    return align256(t * L.Dl * 2) + align256(t * L.Dl * 4) + align256(routed) + align256(t * L.Dl * 4) +
           align256(t * L.Dl * 2) + 2 * align256(t * L.Fs * 4) + align256(t * L.Fs * 2);
}

hipError_t launch_latent(const DevLatent& L, const DevWeights& W, const uint16_t* h, int T, const int32_t* idx,
                         const float* w, int K, float* out, void* ws, hipStream_t stream) {
    rocblas_handle blas = nullptr;
    hipError_t err = blas_for(stream, &blas);
    if (err != hipSuccess) return err;
    const int Dh = L.Dh, Dl = W.D, Fs = L.Fs;
    const size_t t = (size_t)T;
    const size_t routed = T == 1 ? decode_workspace_bytes(K, Dl, W.F) : chunk_workspace_bytes(T, K, W.E, Dl, W.F);
    char* p = static_cast<char*>(ws);
    uint16_t* x = reinterpret_cast<uint16_t*>(p); p += align256(t * Dl * 2);
    float* x32 = reinterpret_cast<float*>(p); p += align256(t * Dl * 4);
    void* rws = p; p += align256(routed);
    float* a = reinterpret_cast<float*>(p); p += align256(t * Dl * 4);
    uint16_t* r = reinterpret_cast<uint16_t*>(p); p += align256(t * Dl * 2);
    float* g = reinterpret_cast<float*>(p); p += align256(t * Fs * 4);
    float* u = reinterpret_cast<float*>(p); p += align256(t * Fs * 4);
    uint16_t* s = reinterpret_cast<uint16_t*>(p);

    // x = Wdn h, then the routed block on x
    err = dense(blas, h, T, Dh, L.w_down, Dl, x, false, 0.0f);
    if (err != hipSuccess) return err;
    if (T == 1) {
        hipLaunchKernelGGL(widen_kernel, dim3(grid_blocks(Dl, 256)), dim3(256), 0, stream, x, Dl, x32);
        err = launch_decode(W, x32, idx, w, K, a, decode_workspace_carve(rws, K, Dl, W.F), stream);
    } else {
        err = launch_chunk(W, x, T, idx, w, K, a, nullptr, chunk_workspace_carve(rws, T, K, W.E, Dl, W.F), stream);
    }
    if (err != hipSuccess) return err;
    // RMSNorm on the aggregate, then back to the full width
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, a, L.norm, Dl, L.eps, r);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = dense(blas, r, T, Dl, L.w_up, Dh, out, true, 0.0f);
    if (err != hipSuccess) return err;
    // the fused shared experts, added into out
    err = dense(blas, h, T, Dh, L.shared_gate, Fs, g, true, 0.0f);
    if (err != hipSuccess) return err;
    err = dense(blas, h, T, Dh, L.shared_up, Fs, u, true, 0.0f);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(situ_kernel, dim3(grid_blocks(t * Fs, 256)), dim3(256), 0, stream, g, u, t * Fs, s);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return dense(blas, s, T, Fs, L.shared_down, Dh, out, true, 1.0f);
}

}  // namespace k3moe
