// decode.hip -- one token through its K routed experts, fp32 end to end.
//
// The routed-expert matmuls of the Kimi K3 engine run straight on the MXFP4 bytes
// (colibri PR #676 summary; PR #684 MXFP4-kernel commit), and decode is bound by
// the expert bytes it streams ("It runs the full model": 25.8 GB of experts per
// token).  Here every selected expert's bytes are read from HBM exactly once:
//
//   kernel 1  per (expert slot k, block of F rows): g_f and u_f for the same f in
//             one wave, SiTU-GLU in registers, h[k, f] to the workspace;
//   kernel 2  per (expert slot k, block of D rows): (W_down h_k)[d] to a partial
//             buffer; the last of the K slot blocks of a row block sums
//             y[d] = sum_k w_k * part[k, d] in slot order (no float atomics, so
//             the result is the same on every run).
//
// Row layout: a row of I inputs is I/32 chunks of 16 packed bytes (= one scale
// group of 32 codes).  Lane l of a wave owns chunks l, l+64, ... and keeps the
// matching activations in registers for all rows the wave visits; each row is a
// coalesced sweep of 16-byte loads, decoded with the gfx950 scaled fp4 converts,
// multiplied in fp32 and reduced across the wave with shuffles.
#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

constexpr int RPW_GU = kDecodeRowsPerWaveGU;
constexpr int RPW_D = kDecodeRowsPerWaveDown;
constexpr int WAVES = kDecodeWaves;

// acc += dot(decode(q, s), xv[0..31])
__device__ __forceinline__ float chunk_dot(uint4 q, uint32_t s, const float* xv, float acc) {
    float wv[8];
    fp4x8_to_f32(q.x, s, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wv[j], xv[j], acc);
    fp4x8_to_f32(q.y, s, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wv[j], xv[8 + j], acc);
    fp4x8_to_f32(q.z, s, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wv[j], xv[16 + j], acc);
    fp4x8_to_f32(q.w, s, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wv[j], xv[24 + j], acc);
    return acc;
}

// Reduce four per-lane values over the wave in 7 shuffles.  On return the total
// of v[0] is in lanes 0..15, v[1] in 16..31, v[2] in 32..47, v[3] in 48..63.
__device__ __forceinline__ float wave_sum4(float v0, float v1, float v2, float v3, int lane) {
    const bool hi32 = lane & 32;
    float a = hi32 ? v2 : v0, b = hi32 ? v3 : v1;  // kept
    float c = hi32 ? v0 : v2, d = hi32 ? v1 : v3;  // sent
    a += __shfl_xor(c, 32, kWave);
    b += __shfl_xor(d, 32, kWave);
    const bool hi16 = lane & 16;
    float keep = hi16 ? b : a, send = hi16 ? a : b;
    keep += __shfl_xor(send, 16, kWave);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) keep += __shfl_xor(keep, off, kWave);
    return keep;
}

template <int CPL>
__device__ __forceinline__ void load_vec_chunks(const float* __restrict__ v, int nch, int lane,
                                                float (&r)[CPL][32]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            const float4* p = reinterpret_cast<const float4*>(v + (size_t)ch * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4 t = p[i];
                r[c][4 * i] = t.x; r[c][4 * i + 1] = t.y; r[c][4 * i + 2] = t.z; r[c][4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) r[c][i] = 0.0f;
        }
    }
}

template <int CPL>
__global__ __launch_bounds__(256, 2) void decode_gateup_kernel(DevWeights W, const float* __restrict__ x,
                                                            const int32_t* __restrict__ idx,
                                                            float* __restrict__ h,
                                                            uint32_t* __restrict__ counters,
                                                            int n_counters) {
    const int k = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the down kernel's arrival counters start at zero for this call
    if (blockIdx.x == 0 && k == 0)
        for (int i = threadIdx.x; i < n_counters; i += blockDim.x) counters[i] = 0u;

    const int D = W.D, F = W.F, nch = D >> 5;
    const int f0 = (blockIdx.x * WAVES + wave) * RPW_GU;
    if (f0 >= F) return;
    const int nf = min(RPW_GU, F - f0);
    float* hk = h + (size_t)k * F;
    const int e = idx[k];
    if (e < 0 || e >= W.E) {
        if (lane < nf) hk[f0 + lane] = __builtin_nanf("");
        return;
    }
    float xr[CPL][32];
    load_vec_chunks<CPL>(x, nch, lane, xr);

    const uint8_t* __restrict__ gq = W.gate_q + (size_t)e * W.gate_q_stride;
    const uint8_t* __restrict__ gs = W.gate_s + (size_t)e * W.gate_s_stride;
    const uint8_t* __restrict__ uq = W.up_q + (size_t)e * W.up_q_stride;
    const uint8_t* __restrict__ us = W.up_s + (size_t)e * W.up_s_stride;
    const size_t qrow = (size_t)D >> 1;

    for (int r = 0; r < nf; r += 2) {
        const int fa = f0 + r;
        const int fb = f0 + min(r + 1, nf - 1);  // duplicate of fa when nf is odd (not stored)
        uint4 qga[CPL], qua[CPL], qgb[CPL], qub[CPL];
        uint32_t sga[CPL], sua[CPL], sgb[CPL], sub[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nch) {
                qga[c] = *reinterpret_cast<const uint4*>(gq + fa * qrow + (size_t)ch * 16);
                qua[c] = *reinterpret_cast<const uint4*>(uq + fa * qrow + (size_t)ch * 16);
                qgb[c] = *reinterpret_cast<const uint4*>(gq + fb * qrow + (size_t)ch * 16);
                qub[c] = *reinterpret_cast<const uint4*>(uq + fb * qrow + (size_t)ch * 16);
                sga[c] = gs[(size_t)fa * nch + ch];
                sua[c] = us[(size_t)fa * nch + ch];
                sgb[c] = gs[(size_t)fb * nch + ch];
                sub[c] = us[(size_t)fb * nch + ch];
            }
        }
        float ag = 0.f, au = 0.f, bg = 0.f, bu = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nch) {
                ag = chunk_dot(qga[c], sga[c], xr[c], ag);
                au = chunk_dot(qua[c], sua[c], xr[c], au);
                bg = chunk_dot(qgb[c], sgb[c], xr[c], bg);
                bu = chunk_dot(qub[c], sub[c], xr[c], bu);
            }
        }
        const float tot = wave_sum4(ag, au, bg, bu, lane);
        // lanes 0 (ag), 16 (au), 32 (bg), 48 (bu): gather the pair for SiTU
        const float g_a = __shfl(tot, 0, kWave), u_a = __shfl(tot, 16, kWave);
        const float g_b = __shfl(tot, 32, kWave), u_b = __shfl(tot, 48, kWave);
        if (lane == 0) hk[fa] = situ_accurate(g_a, u_a);
        if (lane == 1 && r + 1 < nf) hk[fb] = situ_accurate(g_b, u_b);
    }
}

template <int CPL>
__global__ __launch_bounds__(256, 2) void decode_down_kernel(DevWeights W, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ wts, int K,
                                                          const float* __restrict__ h,
                                                          float* __restrict__ ypart,
                                                          uint32_t* __restrict__ counters,
                                                          float* __restrict__ y) {
    __shared__ int s_last;
    const int k = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = W.D, F = W.F, nch = F >> 5;
    const int rows_per_block = WAVES * RPW_D;
    const int d_blk = blockIdx.x * rows_per_block;
    const int d0 = d_blk + wave * RPW_D;
    const int nd = max(0, min(RPW_D, D - d0));
    float* yk = ypart + (size_t)k * D;
    const int e = idx[k];

    if (nd > 0) {
        if (e < 0 || e >= W.E) {
            if (lane < nd) yk[d0 + lane] = __builtin_nanf("");
        } else {
            float hr[CPL][32];
            load_vec_chunks<CPL>(h + (size_t)k * F, nch, lane, hr);
            const uint8_t* __restrict__ dq = W.down_q + (size_t)e * W.down_q_stride;
            const uint8_t* __restrict__ ds = W.down_s + (size_t)e * W.down_s_stride;
            const size_t qrow = (size_t)F >> 1;
            for (int r = 0; r < nd; r += 4) {
                int rr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) rr[i] = d0 + min(r + i, nd - 1);
                uint4 q[4][CPL];
                uint32_t s[4][CPL];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int ch = lane + 64 * c;
                        if (ch < nch) {
                            q[i][c] = *reinterpret_cast<const uint4*>(dq + rr[i] * qrow + (size_t)ch * 16);
                            s[i][c] = ds[(size_t)rr[i] * nch + ch];
                        }
                    }
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + 64 * c;
                    if (ch < nch) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] = chunk_dot(q[i][c], s[i][c], hr[c], acc[i]);
                    }
                }
                const float tot = wave_sum4(acc[0], acc[1], acc[2], acc[3], lane);
                const int i = lane >> 4;
                if ((lane & 15) == 0 && r + i < nd) yk[d0 + r + i] = tot;
            }
        }
    }

    // The last of the K slot blocks for this row block combines, in slot order.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&counters[blockIdx.x], 1u) == (uint32_t)(K - 1));
    __syncthreads();
    if (s_last) {
        __threadfence();
        const int d = d_blk + (int)threadIdx.x;
        if ((int)threadIdx.x < rows_per_block && d < D) {
            float acc = 0.0f;
            for (int k2 = 0; k2 < K; ++k2) acc = fmaf(wts[k2], ypart[(size_t)k2 * D + d], acc);
            y[d] = acc;
        }
    }
}

template <int CPL>
hipError_t launch_gu(const DevWeights& W, const float* x, const int32_t* idx, int K, const DecodeWorkspace& ws,
                     hipStream_t stream) {
    const int rows_per_block = WAVES * RPW_GU;
    dim3 grid((W.F + rows_per_block - 1) / rows_per_block, K);
    hipLaunchKernelGGL(decode_gateup_kernel<CPL>, grid, dim3(WAVES * 64), 0, stream, W, x, idx, ws.h,
                       ws.counters, ws.n_counters);
    return hipGetLastError();
}

template <int CPL>
hipError_t launch_dn(const DevWeights& W, const int32_t* idx, const float* w, int K, float* y,
                     const DecodeWorkspace& ws, hipStream_t stream) {
    dim3 grid(ws.n_counters, K);
    hipLaunchKernelGGL(decode_down_kernel<CPL>, grid, dim3(WAVES * 64), 0, stream, W, idx, w, K, ws.h,
                       ws.ypart, ws.counters, y);
    return hipGetLastError();
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int n_row_blocks_down(int D) { return (D + WAVES * RPW_D - 1) / (WAVES * RPW_D); }

}  // namespace

size_t decode_workspace_bytes(int K, int D, int F) {
    return align256((size_t)K * F * 4) + align256((size_t)K * D * 4) +
           align256((size_t)n_row_blocks_down(D) * 4);
}

DecodeWorkspace decode_workspace_carve(void* ws, int K, int D, int F) {
    char* p = static_cast<char*>(ws);
    DecodeWorkspace r;
    r.h = reinterpret_cast<float*>(p);
    p += align256((size_t)K * F * 4);
    r.ypart = reinterpret_cast<float*>(p);
    p += align256((size_t)K * D * 4);
    r.counters = reinterpret_cast<uint32_t*>(p);
    r.n_counters = n_row_blocks_down(D);
    return r;
}

hipError_t launch_decode(const DevWeights& W, const float* x, const int32_t* idx, const float* w, int K,
                         float* y, const DecodeWorkspace& ws, hipStream_t stream) {
    const int cpl_d = (W.D / 32 + 63) / 64;
    const int cpl_f = (W.F / 32 + 63) / 64;
    hipError_t err;
    switch (cpl_d) {
        case 1: err = launch_gu<1>(W, x, idx, K, ws, stream); break;
        case 2: err = launch_gu<2>(W, x, idx, K, ws, stream); break;
        case 3: err = launch_gu<3>(W, x, idx, K, ws, stream); break;
        default: err = launch_gu<4>(W, x, idx, K, ws, stream); break;
    }
    if (err != hipSuccess) return err;
    switch (cpl_f) {
        case 1: return launch_dn<1>(W, idx, w, K, y, ws, stream);
        case 2: return launch_dn<2>(W, idx, w, K, y, ws, stream);
        case 3: return launch_dn<3>(W, idx, w, K, y, ws, stream);
        default: return launch_dn<4>(W, idx, w, K, y, ws, stream);
    }
}

}  // namespace k3moe
