// decode.hip -- one token through its K routed experts, fp32-accurate.
//
// The routed-expert matmuls of the Kimi K3 engine run straight on the MXFP4 bytes
// (colibri PR #676 summary; PR #684 MXFP4-kernel commit), and decode is bound by
// the expert bytes it streams ("It runs the full model": 25.8 GB of experts per
// token).  Every selected expert's bytes are read from HBM exactly once.
//
// The dot products run on the matrix cores.  Each weight is decoded exactly
// (gfx950 scaled fp4 -> bf16 converts) straight into the B operand of
// v_mfma_f32_16x16x32_bf16.  The fp32 activation vector v is split exactly into
// three bf16 parts v = hi + mid + lo (8 + 8 + 8 significand bits cover fp32's 24),
// which become rows 0..2 of the A operand; rows 3..15 are zero.  Every product
// w * part is exact in fp32 and the MFMA accumulates in fp32, so a row's dot
// product is sum(acc rows 0..2), accurate like an fp32 GEMV while the VALU only
// runs the converts (half an instruction per weight).
//
//   kernel 1  block = (expert slot k, 64 rows of F); wave = 16 rows f: gate and up
//             tiles for the same f, h = SiTU-GLU(g, u) in the epilogue -> h[k, f]
//   kernel 2  block = (expert slot k, 112 rows of D); wave = 16 rows d of W_down
//             against h[k] -> part[k, d]
//   kernel 3  y[d] = sum_k w_k * part[k, d] in slot order (no atomics: the same
//             bits on every run)
//
// Scale bytes are 1/17 of the bytes but, loaded per step, they would double the
// number of cache-line requests; each workgroup instead copies its rows' scale
// bytes (contiguous in memory) into LDS once, and every step reads them there.
//
// Operand layout per 128-column step: lane l = (n = l%16, g = l/16) loads 16 bytes
// = 32 codes = one scale group of weight row n at columns 128s + 32g ... + 31, and
// feeds MFMA j = 0..3 with columns 32g + 8j ... + 7 of that group.  The A operand
// takes the same columns of the activation parts, so each MFMA pairs every
// product exactly once.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

// 4 waves of 16 rows: F = 3072 gives 48 workgroups per slot, 768 for 16 slots,
// exactly three per CU (6-wave workgroups, two per CU, measured slower)
constexpr int WAVES = kDecodeWaves;
constexpr int ROWS_PER_BLOCK = WAVES * 16;
constexpr int PD = 4;                // pipeline depth: steps of weights in flight per wave
// Counters of the down kernel's folded combine: one per block of D rows, 64 words
// apart (one per cache line: device-scope atomics on one line serialize).
constexpr int CNT_STRIDE = 64;

// LDS layout (uint16 elements): [part 0 | part 1 | part 2] each `pstride` long, then
// an 8-element zero block.  pstride = padded columns + 8, so the three parts start
// 4 banks apart.
__host__ __device__ inline int part_stride(int n) { return ((n + 127) & ~127) + 8; }
__host__ __device__ inline size_t parts_lds_bytes(int n) { return (size_t)(3 * part_stride(n) + 8) * 2; }

__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = f32_to_bf16_bits(x);
    const float r1 = x - __uint_as_float(hi << 16);
    mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(mid << 16);
    lo = f32_to_bf16_bits(r2);
}

// Split v (fp32, n a multiple of 32, 16-byte aligned) into three bf16 parts in LDS;
// columns [n, npad) are zero.  Two phases, so a kernel can issue these loads
// first, then its weight prefetch, and only then wait for the activations.
// NT threads stage the vector; each loads up to kMax float4 (8192 columns in all).
template <int NT>
struct Stage {
    static constexpr int kMax = (2048 + NT - 1) / NT;
    float4 r[kMax];
    int n, nits;

    __device__ __forceinline__ void load(const float* __restrict__ v, int n_) {
        n = n_;
        nits = (((n + 127) & ~127) / 4 + NT - 1) / NT;  // block-uniform
#pragma unroll
        for (int it = 0; it < kMax; ++it) {
            const int i4 = min((int)threadIdx.x + it * NT, n / 4 - 1);  // clamped: no branch around the load
            if (it < nits) r[it] = reinterpret_cast<const float4*>(v)[i4];
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds) const {
        const int npad = (n + 127) & ~127, ps = part_stride(n);
#pragma unroll
        for (int it = 0; it < kMax; ++it) {
            const int i = 4 * ((int)threadIdx.x + it * NT);
            if (it < nits && i < npad) {
                const bool in = i < n;
                const float xs[4] = {in ? r[it].x : 0.f, in ? r[it].y : 0.f, in ? r[it].z : 0.f, in ? r[it].w : 0.f};
                uint32_t hi[4], mid[4], lo[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) split3(xs[c], hi[c], mid[c], lo[c]);
                *reinterpret_cast<uint2*>(lds + i) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2*>(lds + ps + i) = make_uint2(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16));
                *reinterpret_cast<uint2*>(lds + 2 * ps + i) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
        if (threadIdx.x < 8) lds[3 * ps + threadIdx.x] = 0;
    }
};

// Branch-free chunk load: columns past kdim read the row's last chunk instead
// (always in bounds); the caller zeroes them with `valid` when the data is used,
// so no load sits behind a branch and the waitcnt pass can keep many in flight.
__device__ __forceinline__ uint4 load_row_chunk(const uint8_t* __restrict__ qrow, int col, int kdim) {
    const int c = min(col, kdim - 32);
    return *reinterpret_cast<const uint4*>(qrow + (c >> 1));
}

// Copy `rows` consecutive scale rows of `sb` bytes (starting at global row r0,
// clamped to nrows) into LDS.  Dword loads when every row is 4-byte aligned.
template <bool DWORD, int ROWS, int NT>
struct ScaleStage {
    // dwords per thread: NT threads x 4 B x kMax >= ROWS rows x 256 B (the widest scale row)
    static constexpr int kMax = (ROWS * 64 + NT - 1) / NT;
    uint32_t v[kMax];
    int nbytes;

    __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int r0, int rows, int nrows, int sb) {
        const int rr = min(rows, nrows - r0);  // rows that exist
        nbytes = rr * sb;
        const uint8_t* p = base + (size_t)r0 * sb;
#pragma unroll
        for (int it = 0; it < kMax; ++it) {
            const int i = (int)threadIdx.x + it * NT;
            if (DWORD) {
                const int c = min(i, nbytes / 4 - 1);
                if (it * NT * 4 < nbytes) v[it] = reinterpret_cast<const uint32_t*>(p)[c];
            } else {
                // byte path: 4 bytes per thread per iteration, assembled in a dword
                uint32_t w = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int c = min(4 * i + b, nbytes - 1);
                    if (it * NT * 4 < nbytes) w |= (uint32_t)p[c] << (8 * b);
                }
                v[it] = w;
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int it = 0; it < kMax; ++it) {
            const int i = (int)threadIdx.x + it * NT;
            if (4 * i < nbytes) *reinterpret_cast<uint32_t*>(lds + 4 * i) = v[it];
        }
    }
};

// One wave's weight stream: NT tiles of 16 rows, PD steps of 128 columns in flight.
template <int NT>
struct RowStream {
    const uint8_t* qrow[NT];
    const uint8_t* srow[NT];  // this lane's row of scale bytes, in LDS
    int kdim;
    uint4 buf[PD][NT];

    // Issue the first PD steps (before anything else, so HBM is busy from the start).
    __device__ __forceinline__ void prefetch() {
        const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int u = 0; u < PD; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t) buf[u][t] = load_row_chunk(qrow[t], u * 128 + 32 * lg, kdim);
    }

    // MFMAs of one step from buffer slot u.
    __device__ __forceinline__ void step(int u, int s, const uint16_t* abase, int astep, int jstep, bool valid,
                                         f32x4 (&acc)[NT]) {
        const uint16_t* ap = abase + s * astep;
        const int lg = (threadIdx.x & 63) >> 4;
        const int sc = min(4 * s + lg, (kdim >> 5) - 1);
        u32x4 b[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint4 q = valid ? buf[u][t] : make_uint4(0u, 0u, 0u, 0u);
            fp4x32_to_bf16(q, srow[t][sc], b[t]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + jstep * j);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b[t][j]), acc[t], 0,
                                                                 0, 0);
        }
    }

    // acc[t] += A(parts) x B(tile t) over all steps; each buffer slot is refilled
    // with the step PD ahead as soon as it is consumed.  A range of columns
    // [col0, col0 + kdim) of a vector staged with part stride ps: qrow and srow
    // then point at the range's first column.
    __device__ __forceinline__ void run(const uint16_t* lds, f32x4 (&acc)[NT], int ps = -1, int col0 = 0) {
        const int lane = threadIdx.x & 63;
        const int ln = lane & 15, lg = lane >> 4;
        const int nsteps = (kdim + 127) >> 7;
        if (ps < 0) ps = part_stride(kdim);
        // A operand: part ln (< 3) at this lane group's columns, or the zero block
        const uint16_t* abase = (ln < 3) ? lds + ln * ps + col0 + 32 * lg : lds + 3 * ps;
        const int astep = (ln < 3) ? 128 : 0;
        const int jstep = (ln < 3) ? 8 : 0;
        int s0 = 0;
        // Slots are refilled in pairs, after the odd step of each pair: an even step
        // and the next one are the two 64-byte halves of each row's 128-byte line, so
        // both halves are requested together (the line is fetched once, whole).
        // Steady state: every refill is in range, so the body has no branches.
        static_assert(PD % 2 == 0, "slots refill in pairs");
        for (; s0 + 2 * PD <= nsteps; s0 += PD) {
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                step(u, s0 + u, abase, astep, jstep, true, acc);
                if (u & 1) {
#pragma unroll
                    for (int v = u - 1; v <= u; ++v)
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            buf[v][t] = load_row_chunk(qrow[t], (s0 + v + PD) * 128 + 32 * lg, kdim);
                }
            }
        }
        // tail: the last PD..2PD-1 steps (only the final step can be partial).  A
        // refill of an even slot needs its odd neighbour's step to exist, which
        // s + PD < nsteps guarantees.
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int s = s0 + u;
            if (s < nsteps) {
                step(u, s, abase, astep, jstep, s * 128 + 32 * lg < kdim, acc);
                if (u & 1) {
#pragma unroll
                    for (int v = u - 1; v <= u; ++v) {
                        if (s0 + v + PD < nsteps) {
#pragma unroll
                            for (int t = 0; t < NT; ++t)
                                buf[v][t] = load_row_chunk(qrow[t], (s0 + v + PD) * 128 + 32 * lg, kdim);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int s = s0 + PD + u;
            if (s < nsteps) step(u, s, abase, astep, jstep, s * 128 + 32 * lg < kdim, acc);
        }
    }
};

// LDS bytes of a decode workgroup: activation parts, then NT x 64 rows of scales
// (+16: the last scale copy may round its final dword up past its rows).
__host__ __device__ inline size_t decode_lds_bytes(int kdim, int nt) {
    return parts_lds_bytes(kdim) + (size_t)nt * ROWS_PER_BLOCK * (kdim / 32) + 16;
}

// Gate/up with pruned slots: the kept slots' rows are served by twice as many
// workgroups of 32 rows, each 16-row tile by two waves that reduce one half of
// the columns each (the second half's sums are added to the first's through
// LDS).  All slots kept: the 64-row workgroups and their summation order.
constexpr int SPLIT_ROWS = ROWS_PER_BLOCK / 2;
constexpr int SPLIT_MERGE_BYTES = 2 * 16 * 8 * 4;  // 2 waves x 16 lanes x 2 tiles x 4 floats
__host__ __device__ inline bool decode_split_ok(int D) { return D % 256 == 0; }

// Rows of one workgroup for slot k and expert e (full: 64 rows [blk*64, +64), four
// waves of 16; SPLIT: 32 rows [blk*32, +32), waves w and w+2 on tile w&1, columns
// [0, D/2) and [D/2, D)).
template <bool DS, bool SPLIT>
__device__ __forceinline__ void gateup_block(const DevWeights& W, const float* __restrict__ x, int e, int k, int blk,
                                             float* __restrict__ h, uint16_t* lds) {
    constexpr int ROWS = SPLIT ? SPLIT_ROWS : ROWS_PER_BLOCK;
    const int lane = threadIdx.x & 63, ln = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = W.D, F = W.F, sb = D >> 5;
    const int fblk = blk * ROWS;
    const int f0 = fblk + (SPLIT ? (wave & 1) : wave) * 16;
    const int half = SPLIT ? (wave >> 1) : 0;
    const int col0 = half * (D / 2);  // first column of this wave's range
    uint8_t* slds = reinterpret_cast<uint8_t*>(lds) + parts_lds_bytes(D);

    if (e == K3MOE_PRUNED) return;  // block-uniform: a pruned slot reads and writes nothing
    const bool valid_e = e >= 0 && e < W.E;
    const int ec = valid_e ? e : 0;

    // activations and scale rows first: waiting for them later leaves the weights in flight
    Stage<WAVES * 64> st;
    st.load(x, D);
    ScaleStage<DS, ROWS, WAVES * 64> sg, su;
    sg.load(W.gate_s + (size_t)ec * W.gate_s_stride, fblk, ROWS, F, sb);
    su.load(W.up_s + (size_t)ec * W.up_s_stride, fblk, ROWS, F, sb);
    // weights: always prefetched (clamped to real rows), so no load sits behind a branch
    const int fc = min(f0, F - 16);
    const size_t qrow = (size_t)D >> 1;
    RowStream<2> rs;
    rs.kdim = SPLIT ? D / 2 : D;
    rs.qrow[0] = W.gate_q + (size_t)ec * W.gate_q_stride + (size_t)(fc + ln) * qrow + (col0 >> 1);
    rs.qrow[1] = W.up_q + (size_t)ec * W.up_q_stride + (size_t)(fc + ln) * qrow + (col0 >> 1);
    rs.srow[0] = slds + (size_t)(fc - fblk + ln) * sb + (col0 >> 5);
    rs.srow[1] = slds + (size_t)(ROWS + fc - fblk + ln) * sb + (col0 >> 5);
    rs.prefetch();
    st.store(lds);
    sg.store(slds);
    su.store(slds + ROWS * sb);
    __syncthreads();
    float* hk = h + (size_t)k * F;
    if (!valid_e) {
        if (f0 < F && lane < 16 && half == 0) hk[f0 + lane] = __builtin_nanf("");
        return;  // block-uniform
    }
    if (!SPLIT && f0 >= F) return;  // no barrier follows
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (SPLIT) {
        rs.run(lds, acc, part_stride(D), col0);
        // the second half's sums to LDS (after the sweep: the merge region follows
        // the scales), then added to the first half's
        float* mrg = reinterpret_cast<float*>(slds + 2 * ROWS * sb + 16);
        if (half == 1 && lane < 16) {
            float* m = mrg + ((wave & 1) * 16 + lane) * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                m[c] = acc[0][c];
                m[4 + c] = acc[1][c];
            }
        }
        __syncthreads();
        if (half == 1 || f0 >= F) return;
        if (lane < 16) {
            const float* m = mrg + ((wave & 1) * 16 + lane) * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[0][c] += m[c];
                acc[1][c] += m[4 + c];
            }
        }
    } else {
        rs.run(lds, acc);
    }
    // C layout: lane l, register r -> row 4*(l/16)+r, column l%16; rows 0..2 are the
    // hi/mid/lo sums of column (= weight row) l for lanes 0..15
    if (lane < 16) {
        const float g = (acc[0][0] + acc[0][1]) + acc[0][2];
        const float u = (acc[1][0] + acc[1][1]) + acc[1][2];
        hk[f0 + lane] = situ_accurate(g, u);
    }
}

// One-dimensional grid of 2*K*nblk workgroups (nblk = 64-row blocks of F).  With
// every slot kept, workgroup g < K*nblk serves slot g / nblk, block g % nblk (the
// rest exit); with some slot pruned (and D a multiple of 256), g < m*2*nblk serves
// the (g / (2*nblk))-th of the m kept slots, 32-row block g % (2*nblk).  split >= 0
// fixes the choice instead (0: 64-row blocks, 1: split when D allows).
template <bool DS>
__global__ __launch_bounds__(WAVES * 64) void decode_gateup_kernel(DevWeights W, const float* __restrict__ x,
                                                            const int32_t* __restrict__ idx, int K, int split,
                                                            float* __restrict__ h, int32_t* __restrict__ cnt,
                                                            int ncnt) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int g = blockIdx.x;
    // the down kernel's combine counters (when folded) start this call at zero
    if (cnt != nullptr && g == 0 && (int)threadIdx.x < ncnt) cnt[threadIdx.x * CNT_STRIDE] = 0;
    const int lane = threadIdx.x & 63;
    const int nblk = (W.F + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    const int kf = min(g / nblk, K - 1);
    const int ef = idx[kf];  // the full-mode expert, loaded beside the kept mask
    const uint64_t keptm = __ballot(lane < K && idx[min(lane, K - 1)] != K3MOE_PRUNED);
    const int m = __popcll(keptm);
    if ((split < 0 ? m == K : split == 0) || !decode_split_ok(W.D)) {
        if (g >= K * nblk) return;
        gateup_block<DS, false>(W, x, ef, kf, g % nblk, h, lds);
        return;
    }
    const int nblk2 = 2 * nblk;
    if (g >= m * nblk2) return;
    // slot of the j-th kept entry
    uint64_t rest = keptm;
    for (int j = g / nblk2; j > 0; --j) rest &= rest - 1;
    const int k = __ffsll((long long)rest) - 1;
    gateup_block<DS, true>(W, x, idx[k], k, g % nblk2, h, lds);
}

constexpr int DOWN_TILES = 1;  // 16-row tiles of W_down per wave
// 7 waves (112 rows): D = 3584 gives 32 workgroups per slot, 512 for 16 slots,
// exactly two per CU (64-row workgroups gave 896, 3.5 per CU: 20.9 against
// 19.6 us; 32-row workgroups, seven per CU: 22.7 us)
constexpr int DOWN_WAVES = 7;
constexpr int DOWN_ROWS_PER_BLOCK = DOWN_WAVES * 16 * DOWN_TILES;

__host__ __device__ inline int down_blocks(int D) { return (D + DOWN_ROWS_PER_BLOCK - 1) / DOWN_ROWS_PER_BLOCK; }

__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every memory operation this wave issued so far has completed (stores included)
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// FOLD: the combine is folded in.  Each workgroup writes its partial rows with
// agent-scope stores, waits until they have completed, and counts itself in its
// block's counter (device-scope atomic); the workgroup that brings the count to
// the number of kept slots has seen every partial of the block completed, and
// forms y there in slot order with agent-scope loads (the same fmaf chain as
// decode_combine_kernel, so the same bits).  The counters start at zero: the
// gate/up kernel of the same call clears them.
template <bool DS, bool FOLD>
__global__ __launch_bounds__(DOWN_WAVES * 64) void decode_down_kernel(DevWeights W, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ h,
                                                          float* __restrict__ ypart, const float* __restrict__ wts,
                                                          int K, float* __restrict__ y, int32_t* __restrict__ cnt) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ int s_last;
    const int k = blockIdx.y;
    const int lane = threadIdx.x & 63, ln = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = W.D, F = W.F, sb = F >> 5;
    const int dblk = blockIdx.x * DOWN_ROWS_PER_BLOCK;
    const int d0 = dblk + wave * 16 * DOWN_TILES;
    const int e = idx[k];
    if (e == K3MOE_PRUNED) {  // block-uniform; a pruned slot is not counted
        if (FOLD && k == 0 && threadIdx.x < 64) {
            // every slot pruned: no workgroup counts, so slot 0's write y = 0 (the
            // combine of no slots)
            const int v = (int)threadIdx.x < K ? idx[threadIdx.x] : K3MOE_PRUNED;
            if (__ballot(v != K3MOE_PRUNED) == 0ull) {
                for (int d = dblk + (int)threadIdx.x; d < min(dblk + DOWN_ROWS_PER_BLOCK, D); d += 64) y[d] = 0.0f;
            }
        }
        return;
    }
    const bool valid_e = e >= 0 && e < W.E;
    const int ec = valid_e ? e : 0;
    uint8_t* slds = reinterpret_cast<uint8_t*>(lds) + parts_lds_bytes(F);

    Stage<DOWN_WAVES * 64> st;
    st.load(h + (size_t)k * F, F);
    ScaleStage<DS, DOWN_ROWS_PER_BLOCK, DOWN_WAVES * 64> sd;
    sd.load(W.down_s + (size_t)ec * W.down_s_stride, dblk, DOWN_ROWS_PER_BLOCK, D, sb);
    const size_t qrow = (size_t)F >> 1;
    RowStream<DOWN_TILES> rs;
    rs.kdim = F;
#pragma unroll
    for (int t = 0; t < DOWN_TILES; ++t) {
        const int dc = min(d0 + 16 * t, D - 16);  // clamped to a real tile
        rs.qrow[t] = W.down_q + (size_t)ec * W.down_q_stride + (size_t)(dc + ln) * qrow;
        rs.srow[t] = slds + (size_t)(dc - dblk + ln) * sb;
    }
    rs.prefetch();
    st.store(lds);
    sd.store(slds);
    __syncthreads();
    float* yk = ypart + (size_t)k * D;
    if constexpr (!FOLD) {
        if (d0 >= D) return;
        if (!valid_e) {
            for (int t = 0; t < DOWN_TILES; ++t)
                if (lane < 16 && d0 + 16 * t < D) yk[d0 + 16 * t + lane] = __builtin_nanf("");
            return;
        }
    }
    float pv[DOWN_TILES];
#pragma unroll
    for (int t = 0; t < DOWN_TILES; ++t) pv[t] = __builtin_nanf("");  // an id out of range: NaN rows
    if (valid_e && d0 < D) {  // wave-uniform
        f32x4 acc[DOWN_TILES];
#pragma unroll
        for (int t = 0; t < DOWN_TILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        rs.run(lds, acc);
#pragma unroll
        for (int t = 0; t < DOWN_TILES; ++t) pv[t] = (acc[t][0] + acc[t][1]) + acc[t][2];
    }
#pragma unroll
    for (int t = 0; t < DOWN_TILES; ++t) {
        if (lane < 16 && d0 + 16 * t < D) {
            if constexpr (FOLD) st_agent(yk + d0 + 16 * t + lane, pv[t]);
            else yk[d0 + 16 * t + lane] = pv[t];
        }
    }
    if constexpr (FOLD) {
        wait_memory();
        __syncthreads();
        if (threadIdx.x < 64) {
            // kept slots of the token (the workgroups that count themselves)
            const int v = (int)threadIdx.x < K ? idx[threadIdx.x] : K3MOE_PRUNED;
            const int m = __popcll(__ballot(v != K3MOE_PRUNED));
            if (threadIdx.x == 0)
                s_last = __hip_atomic_fetch_add(cnt + (size_t)blockIdx.x * CNT_STRIDE, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == m - 1;
        }
        __syncthreads();
        if (s_last && threadIdx.x < DOWN_ROWS_PER_BLOCK) {
            const int d = dblk + (int)threadIdx.x;
            if (d < D) {
                float acc = 0.0f;
                for (int k0 = 0; k0 < K; k0 += 16) {
                    float v[16], wk[16];
                    int id[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {  // the group's loads in flight together
                        const int kk = min(k0 + i, K - 1);
                        id[i] = idx[kk];
                        wk[i] = wts[kk];
                        v[i] = ld_agent(ypart + (size_t)kk * D + d);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (k0 + i < K && id[i] != K3MOE_PRUNED) acc = fmaf(wk[i], v[i], acc);
                }
                y[d] = acc;
            }
        }
    }
}

// y[d] = sum over slots in order of w_k * part[k, d]; pruned slots are skipped.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ ypart,
                                                             const float* __restrict__ wts,
                                                             const int32_t* __restrict__ idx, int K, int D,
                                                             float* __restrict__ y) {
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= D) return;
    float acc = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 16) {
        float v[16], wk[16];
        int id[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // all loads of a group in flight together: the
            const int kk = min(k0 + i, K - 1);  // partials are read whatever the slot
            id[i] = idx[kk];                     // holds (a pruned slot's row is
            wk[i] = wts[kk];                     // workspace memory, never used)
            v[i] = ypart[(size_t)kk * D + d];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (k0 + i < K && id[i] != K3MOE_PRUNED) acc = fmaf(wk[i], v[i], acc);
    }
    y[d] = acc;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t decode_workspace_bytes(int K, int D, int F) {
    return align256((size_t)K * F * 4) + align256((size_t)K * D * 4) + align256((size_t)down_blocks(D) * CNT_STRIDE * 4);
}

DecodeWorkspace decode_workspace_carve(void* ws, int K, int D, int F) {
    char* p = static_cast<char*>(ws);
    DecodeWorkspace r;
    r.h = reinterpret_cast<float*>(p);
    p += align256((size_t)K * F * 4);
    r.ypart = reinterpret_cast<float*>(p);
    p += align256((size_t)K * D * 4);
    r.cnt = reinterpret_cast<int32_t*>(p);
    return r;
}

hipError_t launch_decode_gateup(const DevWeights& W, const float* x, const int32_t* idx, int K, float* h,
                                hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop, int split,
                                int32_t* cnt) {
    const dim3 grid(2 * K * ((W.F + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK));
    const size_t lds = decode_lds_bytes(W.D, 2) + SPLIT_MERGE_BYTES;
    // dword scale copies need every scale row and expert block 4-byte aligned
    const bool dw = (W.D % 128 == 0) && W.gate_s_stride % 4 == 0 && W.up_s_stride % 4 == 0 &&
                    (reinterpret_cast<uintptr_t>(W.gate_s) & 3) == 0 && (reinterpret_cast<uintptr_t>(W.up_s) & 3) == 0;
    const auto kernel = dw ? decode_gateup_kernel<true> : decode_gateup_kernel<false>;
    if (ev_start != nullptr && ev_stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, dim3(WAVES * 64), (uint32_t)lds, stream, ev_start, ev_stop, 0, W, x, idx,
                              K, split, h, cnt, down_blocks(W.D));
    else
        hipLaunchKernelGGL(kernel, grid, dim3(WAVES * 64), lds, stream, W, x, idx, K, split, h, cnt, down_blocks(W.D));
    return hipGetLastError();
}

hipError_t launch_decode_down(const DevWeights& W, const float* h, const int32_t* idx, const float* w, int K,
                              float* ypart, float* y, hipStream_t stream, int32_t* cnt) {
    const dim3 grid(down_blocks(W.D), K);
    const size_t lds = parts_lds_bytes(W.F) + (size_t)DOWN_ROWS_PER_BLOCK * (W.F / 32) + 16;
    const bool dw = (W.F % 128 == 0) && W.down_s_stride % 4 == 0 && (reinterpret_cast<uintptr_t>(W.down_s) & 3) == 0;
    if (cnt != nullptr) {  // combine folded in (the counters were cleared by this call's gate/up kernel)
        const auto kernel = dw ? decode_down_kernel<true, true> : decode_down_kernel<false, true>;
        hipLaunchKernelGGL(kernel, grid, dim3(DOWN_WAVES * 64), lds, stream, W, idx, h, ypart, w, K, y, cnt);
        return hipGetLastError();
    }
    const auto kernel = dw ? decode_down_kernel<true, false> : decode_down_kernel<false, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(DOWN_WAVES * 64), lds, stream, W, idx, h, ypart, w, K, y, cnt);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((W.D + 255) / 256), dim3(256), 0, stream, ypart, w, idx, K, W.D, y);
    return hipGetLastError();
}

hipError_t launch_decode(const DevWeights& W, const float* x, const int32_t* idx, const float* w, int K,
                         float* y, const DecodeWorkspace& ws, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
    hipError_t err = launch_decode_gateup(W, x, idx, K, ws.h, stream, ev_start, ev_stop, -1, ws.cnt);
    if (err != hipSuccess) return err;
    return launch_decode_down(W, ws.h, idx, w, K, ws.ypart, y, stream, ws.cnt);
}

}  // namespace k3moe
