// latent.hip -- the LatentMoE block around the routed experts.
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): latent 7168 <-> 3584
// projections around the experts, RMSNorm on the aggregate, two fused shared
// experts, SiTU-GLU; PR #676 summary: the routed experts run in the latent space
// behind shared down/up projections, plus two fused full-width shared experts.
// Per token with hidden state h [Dh] (bf16):
//   x   = Wdn h                           [Dl]   fp32 (the products' fp32 accumulation;
//                                                nothing is rounded before the experts)
//   a   = sum_k w_k E_k(x)                [Dl]   the routed block: decode GEMVs for one
//                                                token, the grouped chunk GEMMs otherwise
//   r   = gn * a / sqrt(mean(a^2) + eps)  [Dl]   bf16
//   out = Wup r                           [Dh]   fp32
//   g   = Sg h, u = Su h                  [Fs]   fp32
//   s   = SiTU(g, u)                      [Fs]   bf16
//   out += Sd s                           [Dh]
// The five dense products are bf16 x bf16 with fp32 accumulation.  For one token
// they are this file's GEMV kernels (x in one pass with g, u and s, the norm
// folded into the pass that forms out); for a chunk, dense.hip's MFMA kernels
// (x; s with SiTU-GLU in the epilogue; out = Wup r + Sd s as one reduction)
// around the routed chunk path and the rmsnorm kernel.


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

// ------------------------------------------------ one token: bf16 GEMVs
// For a single token the five projections are matrix-vector products that stream
// their bf16 weights once; these kernels do that directly (and fuse what sits
// between them) instead of going through a GEMM library at n = 1:
//   GEMV_X    x = Wdn h in fp32
//   GEMV_SITU s = SiTU(Sg h, Su h) in bf16 (both shared projections in one pass)
//   (the two above run as one launch, gemv_xs_kernel: both read h)
//   out = Wup r + Sd s in fp32, r = RMSNorm(a) computed by every workgroup
//             (same arithmetic as rmsnorm_kernel), in gemv_out_kernel
// Layout: W row-major [O, I] bf16, I a multiple of 32.  A workgroup stages its
// input vectors in LDS as bf16 (zero-padded to whole 512-column chunks); wave w
// owns kGemvRows consecutive rows; lane l reads columns 8l + 512c (16 bytes) of
// each row, four chunks per batch, and accumulates fp32 products in column
// order; a wave sum (fixed order) finishes each dot product.
enum { GEMV_X = 0, GEMV_SITU = 1 };
constexpr int kGemvRows = 1;     // rows per wave
constexpr int kGemvBatch = 4;    // 16-byte chunks per row in flight per lane
constexpr int kGemvRowsPerBlock = 4 * kGemvRows;

struct GemvArgs {
    const uint16_t* W0;  // X: Wdn; SITU: Sg; OUT: Wup
    const uint16_t* W1;  // SITU: Su; OUT: Sd
    int I0, I1;          // widths of the two inputs (SITU: I1 = I0, same input)
    int O;               // rows
    const uint16_t* v0;  // X, SITU: h (bf16)
    const float* a;      // OUT: routed aggregate (fp32 [I0]) ...
    const uint16_t* gn;  //      ... and the RMSNorm weight (bf16 [I0])
    float eps;
    const uint16_t* v1;  // OUT: s (bf16 [I1])
    uint16_t* yb;        // SITU: s bf16
    float* yf;           // X: x fp32; OUT: out
};

__host__ __device__ inline int gemv_pad(int n) { return (n + 511) & ~511; }

// v (bf16, n values) -> LDS, zero past n up to the padded width
__device__ __forceinline__ void gemv_stage(const uint16_t* __restrict__ v, int n, uint16_t* dst) {
    const int np = gemv_pad(n);
    for (int i = 8 * (int)threadIdx.x; i < np; i += 8 * 256) {
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (i < n) q = *reinterpret_cast<const uint4*>(v + i);
        *reinterpret_cast<uint4*>(dst + i) = q;
    }
}

__device__ __forceinline__ float dot8_bf16(const u32x4& w, const uint4& v, float acc) {
    acc = fmaf(__uint_as_float(w.x << 16), __uint_as_float(v.x << 16), acc);
    acc = fmaf(__uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(v.x & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(w.y << 16), __uint_as_float(v.y << 16), acc);
    acc = fmaf(__uint_as_float(w.y & 0xFFFF0000u), __uint_as_float(v.y & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(w.z << 16), __uint_as_float(v.z << 16), acc);
    acc = fmaf(__uint_as_float(w.z & 0xFFFF0000u), __uint_as_float(v.z & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(w.w << 16), __uint_as_float(v.w << 16), acc);
    acc = fmaf(__uint_as_float(w.w & 0xFFFF0000u), __uint_as_float(v.w & 0xFFFF0000u), acc);
    return acc;
}

typedef u32x4 GemvBatch[kGemvRows][kGemvBatch];

// Issue the loads of batch c0 (chunks c0 .. c0 + kGemvBatch - 1) of the rows, all
// before any use.  Chunks past the row (the batch's tail, or a lane past a width
// that is not a multiple of 512) load an in-range address and are replaced by
// zeros, so the body has no branches.
__device__ __forceinline__ void gemv_issue(const uint16_t* __restrict__ W, int I, const int (&rows)[kGemvRows],
                                           int c0, GemvBatch& w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
        for (int b = 0; b < kGemvBatch; ++b) {
            const int col = 8 * lane + 512 * (c0 + b);
            const u32x4 q = *reinterpret_cast<const u32x4*>(W + (size_t)rows[r] * I + min(col, I - 8));
            w[r][b] = col < I ? q : u32x4{0u, 0u, 0u, 0u};
        }
}

// acc[r] += W[rows[r], :] . v over the lane's chunks (v in LDS, zero-padded to
// whole chunks, so chunks past the row meet zeros on both sides).  The first
// batch's loads were issued by the caller (pre), before it staged v, so the
// weight stream starts with the kernel.
__device__ __forceinline__ void gemv_rows(const uint16_t* __restrict__ W, int I, const int (&rows)[kGemvRows],
                                          const uint16_t* v, float (&acc)[kGemvRows], const GemvBatch& pre) {
    const int lane = threadIdx.x & 63;
    const int nch = gemv_pad(I) / 512;
    for (int c0 = 0; c0 < nch; c0 += kGemvBatch) {
        GemvBatch w;
        if (c0 == 0) {
#pragma unroll
            for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
                for (int b = 0; b < kGemvBatch; ++b) w[r][b] = pre[r][b];
        } else {
            gemv_issue(W, I, rows, c0, w);
        }
#pragma unroll
        for (int b = 0; b < kGemvBatch; ++b) {
            const bool in = c0 + b < nch;
            uint4 vv = *reinterpret_cast<const uint4*>(v + 8 * lane + 512 * min(c0 + b, nch - 1));
            if (!in) vv = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int r = 0; r < kGemvRows; ++r) acc[r] = dot8_bf16(w[r][b], vv, acc[r]);
        }
    }
}

// The wave's rows of workgroup blk (clamped to real rows) and the first batch of
// their W0 chunks, issued before the workgroup stages its inputs.
struct GemvRows {
    int o0;
    int rows[kGemvRows];
    GemvBatch pre;
};
__device__ __forceinline__ void gemv_prefetch(const GemvArgs& g, int blk, GemvRows& wr) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    wr.o0 = blk * kGemvRowsPerBlock + wave * kGemvRows;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) wr.rows[r] = min(wr.o0 + r, g.O - 1);
    gemv_issue(g.W0, g.I0, wr.rows, 0, wr.pre);
}

// One GEMV workgroup's rows [blk * kGemvRowsPerBlock, ...) once its input is in
// LDS (vs: v0 padded).
template <int EPI>
__device__ __forceinline__ void gemv_block_rows(const GemvArgs& g, const uint16_t* vs, const GemvRows& wr) {
    const int o0 = wr.o0;
    if (o0 >= g.O) return;  // wave-uniform; no barrier follows
    float acc0[kGemvRows] = {}, acc1[kGemvRows] = {};
    gemv_rows(g.W0, g.I0, wr.rows, vs, acc0, wr.pre);
    if (EPI == GEMV_SITU) {
        GemvBatch p1;
        gemv_issue(g.W1, g.I0, wr.rows, 0, p1);
        gemv_rows(g.W1, g.I0, wr.rows, vs, acc1, p1);
    }
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
        const float d0 = wave_sum(acc0[r]);
        const float d1 = (EPI == GEMV_X) ? 0.f : wave_sum(acc1[r]);
        const int o = o0 + r;
        if (lane != 0 || o >= g.O) continue;
        if (EPI == GEMV_X)
            g.yf[o] = d0;
        else
            g.yb[o] = (uint16_t)f32_to_bf16_bits(situ_fast(d0, d1));
    }
}

// x = Wdn h and s = SiTU(Sg h, Su h) in one launch: both read h, so one grid
// stages h once per workgroup and the two projections share one ramp and one
// tail.  Workgroups [0, nbs) take rows of s (the heavier ones first), the rest
// rows of x.
__global__ __launch_bounds__(256) void gemv_xs_kernel(GemvArgs gx, GemvArgs gs, int nbs) {
    extern __shared__ __attribute__((aligned(16))) uint16_t vs[];
    const int b = blockIdx.x;
    GemvRows wr;
    if (b < nbs)
        gemv_prefetch(gs, b, wr);
    else
        gemv_prefetch(gx, b - nbs, wr);
    gemv_stage(gx.v0, gx.I0, vs);
    __syncthreads();
    if (b < nbs)
        gemv_block_rows<GEMV_SITU>(gs, vs, wr);
    else
        gemv_block_rows<GEMV_X>(gx, vs, wr);
}

// out = Wup r + Sd s with r = RMSNorm(a), computed by every workgroup with the
// same arithmetic as rmsnorm_kernel.  The S_d product needs only s, so it runs
// first, while the loads of a are in flight; the norm, its barriers and the W_up
// product follow, the first W_up batch issued before them.  d0 (W_up r) and d1
// (S_d s) are each summed exactly as before and added as d0 + d1.
__global__ __launch_bounds__(256) void gemv_out_kernel(GemvArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint16_t vs[];  // r (padded), then s (padded)
    __shared__ float part[256 / kWave];
    uint16_t* vs1 = vs + gemv_pad(g.I0);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int o0 = blockIdx.x * kGemvRowsPerBlock + wave * kGemvRows;
    int rows[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) rows[r] = min(o0 + r, g.O - 1);
    GemvBatch pre1;
    gemv_issue(g.W1, g.I1, rows, 0, pre1);
    const float4* arow = reinterpret_cast<const float4*>(g.a);
    const int n4 = g.I0 >> 2;
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        v[j] = i < n4 ? arow[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    gemv_stage(g.v1, g.I1, vs1);
    __syncthreads();
    float acc0[kGemvRows] = {}, acc1[kGemvRows] = {};
    if (o0 < g.O) gemv_rows(g.W1, g.I1, rows, vs1, acc1, pre1);  // wave-uniform
    GemvBatch pre0;
    gemv_issue(g.W0, g.I0, rows, 0, pre0);
    // RMSNorm of a, exactly as rmsnorm_kernel: sum of squares in the same order,
    // r = bf16(gn * (a * inv))
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < 256 / kWave; ++j) tot += part[j];
    const float inv = 1.0f / sqrtf(tot / (float)g.I0 + g.eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        if (i >= n4) break;
        const uint2 gw = reinterpret_cast<const uint2*>(g.gn)[i];
        const float g0 = __uint_as_float(gw.x << 16), g1 = __uint_as_float(gw.x & 0xFFFF0000u);
        const float g2 = __uint_as_float(gw.y << 16), g3 = __uint_as_float(gw.y & 0xFFFF0000u);
        reinterpret_cast<uint2*>(vs)[i] = make_uint2(pack_bf16x2(g0 * (v[j].x * inv), g1 * (v[j].y * inv)),
                                                     pack_bf16x2(g2 * (v[j].z * inv), g3 * (v[j].w * inv)));
    }
    for (int i = g.I0 + (int)threadIdx.x; i < gemv_pad(g.I0); i += 256) vs[i] = 0;
    __syncthreads();
    if (o0 >= g.O) return;  // wave-uniform; no barrier follows
    gemv_rows(g.W0, g.I0, rows, vs, acc0, pre0);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
        const float d0 = wave_sum(acc0[r]);
        const float d1 = wave_sum(acc1[r]);
        const int o = o0 + r;
        if (lane == 0 && o < g.O) g.yf[o] = d0 + d1;
    }
}

hipError_t launch_gemv_out(const GemvArgs& g, hipStream_t stream) {
    const size_t lds = (size_t)(gemv_pad(g.I0) + gemv_pad(g.I1)) * 2;
    const dim3 grid((g.O + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock);
    hipLaunchKernelGGL(gemv_out_kernel, grid, dim3(256), lds, stream, g);
    return hipGetLastError();
}

hipError_t launch_gemv_xs(const GemvArgs& gx, const GemvArgs& gs, hipStream_t stream) {
    const size_t lds = (size_t)gemv_pad(gx.I0) * 2;
    const int nbs = (gs.O + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
    const int nbx = (gx.O + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
    hipLaunchKernelGGL(gemv_xs_kernel, dim3(nbs + nbx), dim3(256), lds, stream, gx, gs, nbs);
    return hipGetLastError();
}


}  // namespace

// x (fp32), the routed block's workspace, a, r, s; for T >= 2 the dense products'
// split partials and their counters (three launches).
size_t latent_workspace_bytes(const LatentDims& L, int T, int K, int E) {
    const size_t t = (size_t)T;
    const size_t routed = T == 1 ? decode_workspace_bytes(K, L.Dl, L.F) : chunk_workspace_bytes(T, K, E, L.Dl, L.F);
    const size_t dense = T == 1 ? 0 : align256(dense_part_bytes(T)) + 3 * align256(dense_cnt_bytes());
    return align256(t * L.Dl * 4) + align256(routed) + align256(t * L.Dl * 4) + align256(t * L.Dl * 2) +
           align256(t * L.Fs * 2) + dense;
}

hipError_t launch_latent(const DevLatent& L, const DevWeights& W, const uint16_t* h, int T, const int32_t* idx,
                         const float* w, int K, float* out, void* ws, hipStream_t stream) {
    hipError_t err = hipSuccess;
    const int Dh = L.Dh, Dl = W.D, Fs = L.Fs;
    const size_t t = (size_t)T;
    const size_t routed = T == 1 ? decode_workspace_bytes(K, Dl, W.F) : chunk_workspace_bytes(T, K, W.E, Dl, W.F);
    char* p = static_cast<char*>(ws);
    float* x32 = reinterpret_cast<float*>(p); p += align256(t * Dl * 4);
    void* rws = p; p += align256(routed);
    float* a = reinterpret_cast<float*>(p); p += align256(t * Dl * 4);
    uint16_t* r = reinterpret_cast<uint16_t*>(p); p += align256(t * Dl * 2);
    uint16_t* s = reinterpret_cast<uint16_t*>(p); p += align256(t * Fs * 2);

    if (T == 1) {
        // one token: x = Wdn h (fp32), s = SiTU(Sg h, Su h), the routed decode path
        // on x, then out = Wup RMSNorm(a) + Sd s
        GemvArgs gx{};
        gx.W0 = L.w_down; gx.I0 = Dh; gx.O = Dl; gx.v0 = h; gx.yf = x32;
        GemvArgs gs{};
        gs.W0 = L.shared_gate; gs.W1 = L.shared_up; gs.I0 = Dh; gs.I1 = Dh; gs.O = Fs; gs.v0 = h; gs.yb = s;
        err = launch_gemv_xs(gx, gs, stream);
        if (err != hipSuccess) return err;
        err = launch_decode(W, x32, idx, w, K, a, decode_workspace_carve(rws, K, Dl, W.F), stream);
        if (err != hipSuccess) return err;
        GemvArgs go{};
        go.W0 = L.w_up; go.W1 = L.shared_down; go.I0 = Dl; go.I1 = Fs; go.O = Dh;
        go.a = a; go.gn = L.norm; go.eps = L.eps; go.v1 = s; go.yf = out;
        return launch_gemv_out(go, stream);
    }
    // T >= 2: the dense products on this library's MFMA kernels (dense.hip)
    float* part = reinterpret_cast<float*>(p); p += align256(dense_part_bytes(T));
    int32_t* cnt = reinterpret_cast<int32_t*>(p);
    const size_t cstride = align256(dense_cnt_bytes()) / sizeof(int32_t);
    err = launch_dense_clear(cnt, 3, stream);
    if (err != hipSuccess) return err;
    // x = Wdn h in fp32, s = SiTU(Sg h, Su h) in bf16
    DenseProblem px{};
    px.epi = DENSE_F32; px.A[0] = h; px.W[0] = L.w_down; px.K[0] = Dh; px.T = T; px.N = Dl; px.outf = x32;
    err = launch_dense(px, part, cnt, stream);
    if (err != hipSuccess) return err;
    DenseProblem ps{};
    ps.epi = DENSE_SITU; ps.A[0] = h; ps.W[0] = L.shared_gate; ps.Wu = L.shared_up; ps.K[0] = Dh; ps.T = T;
    ps.N = Fs; ps.outb = s;
    err = launch_dense(ps, part, cnt + cstride, stream);
    if (err != hipSuccess) return err;
    // the routed block on x
    err = launch_chunk(W, x32, nullptr, T, idx, w, K, a, nullptr, chunk_workspace_carve(rws, T, K, W.E, Dl, W.F),
                       stream);
    if (err != hipSuccess) return err;
    // RMSNorm on the aggregate, then out = Wup r + Sd s in one reduction
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, a, L.norm, Dl, L.eps, r);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    DenseProblem po{};
    po.epi = DENSE_F32; po.A[0] = r; po.W[0] = L.w_up; po.K[0] = Dl; po.A[1] = s; po.W[1] = L.shared_down;
    po.K[1] = Fs; po.T = T; po.N = Dh; po.outf = out;
    return launch_dense(po, part, cnt + 2 * cstride, stream);
}

}  // namespace k3moe
