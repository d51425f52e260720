// chunk.hip -- a chunk of tokens through the routed experts, expert union deduplicated.
//
// colibri PR #676, chunked-prefill paragraph: within a chunk the MoE loads each
// unique expert once and runs it for every position routed to it; PR #684,
// chunked-prefill commit: the position lists come from a counting sort.  On the
// GPU the union turns the per-token GEMVs into a grouped matrix product whose
// weight operand is each routed expert's MXFP4 bytes, streamed once per tile of
// up to 128 of its pairs.
//
// Kernels, in stream order (x arrives as bf16):
//   group_count    per 64-token block: one 64-bit mask per expert (bit i = token
//                  t0+i chose it); popcounts are the block's per-expert counts
//   group_scan     one workgroup: per-expert totals, offsets, the union list,
//                  and the GEMM tile list (expert, first row, rows)
//   group_scatter  pair p = t*K+k goes to offsets[e] + (pairs of e in earlier
//                  blocks) + popcount(mask & bits below t): a stable counting sort
//   gemm<GATEUP>   h = SiTU(x W_gate^T, x W_up^T) per tile, bf16 MFMA, h in bf16
//   gemm<DOWN>     y_pair = w_pair * (h W_down^T), fp32, at row p = t*K+k
//   combine        y_t = sum_k y_pair[t*K+k] in slot order
//
// GEMM structure (gfx950, v_mfma_f32_16x16x32_bf16, wave64):
//   workgroup = 4 waves = one (tile, column block); the tile's rows of A
//   (activations, shared by the 4 waves) are staged in LDS 128 columns at a time
//   with the next step prefetched in registers.  The weight operand never
//   touches LDS: each lane loads 16 bytes (32 codes = one scale group) of one
//   weight row and converts them with the gfx950 scaled fp4->bf16 converts
//   straight into four MFMA B operands.  The k order inside a 128-wide step is
//   permuted (lane group g owns columns 32g..32g+31, MFMA j takes 8j..8j+7 of
//   them) identically for A and B, which leaves the dot products unchanged.
//   Workgroup ids are remapped so each XCD walks a contiguous run of
//   (tile, column block) items: the column blocks of one tile share that XCD's L2
//   copy of the tile's activations.
#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

constexpr int GT = kGroupTokens;
constexpr int MT = kTileRows;
constexpr int KS = 128;                 // reduction columns per pipeline step
constexpr int LDS_STRIDE = KS * 2 + 16; // bytes per staged A row (pad staggers banks)
constexpr int GEMM_THREADS = 256;
constexpr int N_XCD = 8;

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// ------------------------------------------------------------------------ grouping
__global__ __launch_bounds__(256) void group_count_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                          int E, int32_t* __restrict__ counts_blk,
                                                          unsigned long long* __restrict__ masks_blk,
                                                          int32_t* __restrict__ err_blk) {
    extern __shared__ unsigned long long smask[];  // [E]
    __shared__ int s_err;
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) smask[e] = 0ull;
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
    const int t0 = b * GT, t1 = min(T, t0 + GT);
    for (int p = t0 * K + (int)threadIdx.x; p < t1 * K; p += blockDim.x) {
        const int e = idx[p];
        if (e < 0 || e >= E) {
            atomicOr(&s_err, 1);
            continue;
        }
        const unsigned long long bit = 1ull << (p / K - t0);
        const unsigned long long old = atomicOr(&smask[e], bit);
        if (old & bit) atomicOr(&s_err, 1);  // one token lists this expert twice
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const unsigned long long m = smask[e];
        counts_blk[(size_t)b * E + e] = __popcll(m);
        masks_blk[(size_t)b * E + e] = m;
    }
    if (threadIdx.x == 0) err_blk[b] = s_err;
}

// Inclusive scan over the 1024 threads of the block of three values at once.
__device__ __forceinline__ void block_scan3(int& a, int& b, int& c, int (*wtot)[16]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int ta = __shfl_up(a, off, kWave), tb = __shfl_up(b, off, kWave), tc = __shfl_up(c, off, kWave);
        if (lane >= off) { a += ta; b += tb; c += tc; }
    }
    if (lane == 63) { wtot[0][wave] = a; wtot[1][wave] = b; wtot[2][wave] = c; }
    __syncthreads();
    if (threadIdx.x < 16) {
        int x0 = wtot[0][threadIdx.x], x1 = wtot[1][threadIdx.x], x2 = wtot[2][threadIdx.x];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int y0 = __shfl_up(x0, off, kWave), y1 = __shfl_up(x1, off, kWave), y2 = __shfl_up(x2, off, kWave);
            if ((int)threadIdx.x >= off) { x0 += y0; x1 += y1; x2 += y2; }
        }
        wtot[0][threadIdx.x] = x0; wtot[1][threadIdx.x] = x1; wtot[2][threadIdx.x] = x2;
    }
    __syncthreads();
    if (wave > 0) { a += wtot[0][wave - 1]; b += wtot[1][wave - 1]; c += wtot[2][wave - 1]; }
}

__global__ __launch_bounds__(1024) void group_scan_kernel(int T, int K, int E, int nb,
                                                          const int32_t* __restrict__ counts_blk,
                                                          int32_t* __restrict__ blkoff,
                                                          const int32_t* __restrict__ err_blk,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ uniq,
                                                          int4* __restrict__ tiles, int max_tiles,
                                                          int32_t* __restrict__ scalars,
                                                          int32_t* __restrict__ n_unique_out) {
    extern __shared__ int32_t scnt[];  // [E]
    __shared__ int wtot[3][16];
    __shared__ int s_err;
    const int tid = threadIdx.x;
    if (tid == 0) {
        int err = 0;
        for (int b = 0; b < nb; ++b) err |= err_blk[b];
        s_err = err;
    }
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int b = 0; b < nb; ++b) {
            const int c = counts_blk[(size_t)b * E + e];
            blkoff[(size_t)b * E + e] = run;  // pairs of e in earlier token blocks
            run += c;
        }
        scnt[e] = run;
        counts[e] = run;
    }
    __syncthreads();

    const int ept = (E + (int)blockDim.x - 1) / (int)blockDim.x;  // experts per thread
    const int e0 = min(E, tid * ept), e1 = min(E, e0 + ept);
    int c = 0, u = 0, nt = 0;
    for (int e = e0; e < e1; ++e) {
        c += scnt[e];
        u += scnt[e] > 0;
        nt += (scnt[e] + MT - 1) / MT;
    }
    int ci = c, ui = u, nti = nt;
    block_scan3(ci, ui, nti, wtot);
    int off = ci - c, upos = ui - u, tpos = nti - nt;  // exclusive prefixes
    for (int e = e0; e < e1; ++e) {
        const int n = scnt[e];
        offsets[e] = off;
        if (n > 0) uniq[upos++] = e;
        for (int j = 0; j * MT < n; ++j, ++tpos)
            if (tpos < max_tiles) tiles[tpos] = make_int4(e, off + j * MT, min(MT, n - j * MT), 0);
        off += n;
    }
    if (tid == (int)blockDim.x - 1) {
        offsets[E] = ci;
        const int nu = s_err ? -1 : ui;
        scalars[0] = nu;
        scalars[1] = s_err ? 0 : min(nti, max_tiles);
        if (n_unique_out) *n_unique_out = nu;
    }
}

__global__ __launch_bounds__(256) void group_scatter_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                            int E,
                                                            const unsigned long long* __restrict__ masks_blk,
                                                            const int32_t* __restrict__ blkoff,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ scalars,
                                                            int32_t* __restrict__ perm) {
    if (scalars[0] < 0) return;  // invalid routing: nothing is placed
    const int b = blockIdx.x;
    const int t0 = b * GT, t1 = min(T, t0 + GT);
    for (int p = t0 * K + (int)threadIdx.x; p < t1 * K; p += blockDim.x) {
        const int e = idx[p];
        const int ti = p / K - t0;
        const unsigned long long m = masks_blk[(size_t)b * E + e];
        const int rank = __popcll(m & ((1ull << ti) - 1ull));
        perm[offsets[e] + blkoff[(size_t)b * E + e] + rank] = p;
    }
}

// ----------------------------------------------------------------------------- GEMM
enum { GATEUP = 0, DOWN = 1 };

struct GemmArgs {
    const uint16_t* A;      // GATEUP: x bf16 [T, Kdim] by token; DOWN: h bf16 [P, Kdim] by grouped row
    const int32_t* perm;    // grouped row -> pair id
    int K;                  // slots per token
    const uint8_t *q0, *s0, *q1, *s1;  // GATEUP: gate, up; DOWN: down (q1/s1 unused)
    int64_t q0_stride, s0_stride, q1_stride, s1_stride;
    int Kdim;               // reduction length
    int N;                  // output columns per expert
    const int4* tiles;
    const int32_t* scalars;  // [1] = number of tiles
    int nblk_n;             // column blocks
    uint16_t* h_out;        // GATEUP output [P, N] bf16, grouped rows
    float* y_out;           // DOWN output [P, N] fp32, pair rows
    const float* wts;       // DOWN: [P] routing weight of each pair
};

template <int MODE>
__global__ __launch_bounds__(GEMM_THREADS, 1) void gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[MT * LDS_STRIDE];

    // ---- work item (XCD-aware): XCD x walks items [x*per, (x+1)*per)
    const int n_items = a.scalars[1] * a.nblk_n;
    const int xcd = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD;
    const int per = (n_items + N_XCD - 1) / N_XCD;
    const int item = xcd * per + slot;
    if (slot >= per || item >= n_items) return;  // block-uniform
    const int tile = item / a.nblk_n, nblk = item % a.nblk_n;
    const int4 td = a.tiles[tile];
    const int e = td.x, row0 = td.y, mrows = td.z;
    const int msub = (mrows + 15) >> 4;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lg = lane >> 4;

    // ---- this wave's output columns
    constexpr int WN = (MODE == GATEUP) ? 32 : 64;   // per gate/up pair (GATEUP) or plain
    const int n0 = nblk * (4 * WN) + wave * WN;
    const int nvalid = min(WN, a.N - n0);             // multiple of 16 (N % 32 == 0)
    const int nsub = (MODE == GATEUP) ? (nvalid > 0 ? 4 : 0) : max(0, nvalid >> 4);

    // ---- B row pointers for the 4 n-subtiles of this lane
    const size_t qrow = (size_t)a.Kdim >> 1, srow = (size_t)a.Kdim >> 5;
    const uint8_t* bq[4];
    const uint8_t* bs[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        int row;
        const uint8_t *q, *s;
        if (MODE == GATEUP) {
            row = n0 + 16 * (ns & 1) + ln;
            q = (ns < 2) ? a.q0 + (size_t)e * a.q0_stride : a.q1 + (size_t)e * a.q1_stride;
            s = (ns < 2) ? a.s0 + (size_t)e * a.s0_stride : a.s1 + (size_t)e * a.s1_stride;
        } else {
            row = n0 + 16 * ns + ln;
            q = a.q0 + (size_t)e * a.q0_stride;
            s = a.s0 + (size_t)e * a.s0_stride;
        }
        row = min(row, a.N - 1);  // clamp for idle subtiles (never used)
        bq[ns] = q + (size_t)row * qrow;
        bs[ns] = s + (size_t)row * srow;
    }

    // ---- A rows this thread stages: rows r = (tid>>4) + 16*pass, 16-byte segment tid&15
    const int seg = tid & 15, rbase = tid >> 4;
    const uint16_t* arow[MT / 16];
#pragma unroll
    for (int pass = 0; pass < MT / 16; ++pass) {
        const int r = rbase + 16 * pass;
        arow[pass] = nullptr;
        if (r < mrows) {
            const size_t row = (MODE == GATEUP) ? (size_t)(a.perm[row0 + r] / a.K) : (size_t)(row0 + r);
            arow[pass] = a.A + row * (size_t)a.Kdim;
        }
    }

    const int nsteps = (a.Kdim + KS - 1) / KS;
    uint4 areg[MT / 16];
    auto load_a = [&](int step) {
        const int kc = step * KS + seg * 8;
#pragma unroll
        for (int pass = 0; pass < MT / 16; ++pass) {
            areg[pass] = make_uint4(0u, 0u, 0u, 0u);
            if (arow[pass] != nullptr && kc < a.Kdim)
                areg[pass] = *reinterpret_cast<const uint4*>(arow[pass] + kc);
        }
    };
    auto store_a = [&]() {
#pragma unroll
        for (int pass = 0; pass < MT / 16; ++pass) {
            const int r = rbase + 16 * pass;
            if (r < mrows) *reinterpret_cast<uint4*>(lds + r * LDS_STRIDE + seg * 16) = areg[pass];
        }
    };

    uint4 bcur[4], bnext[4];
    uint32_t scur[4], snext[4];
    auto load_b = [&](int step, uint4 (&q)[4], uint32_t (&s)[4]) {
        const int kc = step * KS + 32 * lg;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            q[ns] = make_uint4(0u, 0u, 0u, 0u);
            s[ns] = 127u;
            if (ns < nsub && kc < a.Kdim) {
                q[ns] = *reinterpret_cast<const uint4*>(bq[ns] + (kc >> 1));
                s[ns] = bs[ns][kc >> 5];
            }
        }
    };

    f32x4 acc[MT / 16][4];
#pragma unroll
    for (int i = 0; i < MT / 16; ++i)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[i][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_b(0, bcur, scur);
    store_a();
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
        const bool more = step + 1 < nsteps;
        if (more) {
            load_a(step + 1);
            load_b(step + 1, bnext, snext);
        }
        if (nsub > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x8 bop[4];
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) {
                    const uint32_t qw = (j == 0) ? bcur[ns].x : (j == 1) ? bcur[ns].y : (j == 2) ? bcur[ns].z : bcur[ns].w;
                    bop[ns] = __builtin_bit_cast(bf16x8, fp4x8_to_bf16(qw, scur[ns]));
                }
#pragma unroll
                for (int i = 0; i < MT / 16; ++i) {
                    if (i < msub) {
                        const bf16x8 aop = *reinterpret_cast<const bf16x8*>(
                            lds + (16 * i + ln) * LDS_STRIDE + 64 * lg + 16 * j);
#pragma unroll
                        for (int ns = 0; ns < 4; ++ns)
                            if (ns < nsub)
                                acc[i][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[ns], acc[i][ns], 0, 0, 0);
                    }
                }
            }
        }
        if (more) {
            __syncthreads();
            store_a();
            __syncthreads();
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) { bcur[ns] = bnext[ns]; scur[ns] = snext[ns]; }
        }
    }

    // ---- epilogue.  C layout: lane l, register r -> row 4*(l/16)+r, column l%16.
    if (nsub == 0) return;
#pragma unroll
    for (int i = 0; i < MT / 16; ++i) {
        if (i >= msub) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m >= mrows) continue;
            if (MODE == GATEUP) {
                uint16_t* hrow = a.h_out + (size_t)(row0 + m) * a.N;
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const float hv = situ_fast(acc[i][ns][r], acc[i][ns + 2][r]);
                    hrow[n0 + 16 * ns + ln] = (uint16_t)f32_to_bf16_bits(hv);
                }
            } else {
                const int p = a.perm[row0 + m];
                const float wp = a.wts[p];
                float* yrow = a.y_out + (size_t)p * a.N;
#pragma unroll
                for (int ns = 0; ns < 4; ++ns)
                    if (ns < nsub) yrow[n0 + 16 * ns + ln] = acc[i][ns][r] * wp;
            }
        }
    }
}

// -------------------------------------------------------------------------- combine
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ytk, int T, int K, int D,
                                                      const int32_t* __restrict__ scalars,
                                                      float* __restrict__ y) {
    const bool bad = scalars[0] < 0;
    const size_t n4 = (size_t)T * D / 4;
    const int d4 = D / 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const size_t t = i / d4, dd = i % d4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (bad) {
            const float nan = __builtin_nanf("");
            acc = make_float4(nan, nan, nan, nan);
        } else {
            for (int k = 0; k < K; ++k) {
                const float4 v = reinterpret_cast<const float4*>(ytk + ((t * K + k) * (size_t)D))[dd];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
        }
        reinterpret_cast<float4*>(y)[i] = acc;
    }
}

int grid_for(size_t n, int per_block) {
    size_t b = (n + per_block - 1) / per_block;
    return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

// ------------------------------------------------------------------ workspace layout
int group_max_tiles(int T, int K, int E) {
    const long P = (long)T * K;
    return (int)((P + MT - 1) / MT + (E < P ? E : P));
}

size_t group_workspace_bytes(int T, int K, int E, bool with_outputs) {
    const size_t nb = (size_t)(T + GT - 1) / GT;
    size_t b = align256(nb * E * 4) + align256(nb * E * 8) + align256(nb * E * 4) + align256(nb * 4) +
               align256(2 * 4) + align256((size_t)group_max_tiles(T, K, E) * 16);
    if (with_outputs)
        b += align256((size_t)E * 4) + align256((size_t)(E + 1) * 4) + align256((size_t)T * K * 4) +
             align256((size_t)E * 4);
    return b;
}

GroupBuffers group_workspace_carve(void* ws, int T, int K, int E, bool with_outputs) {
    char* p = static_cast<char*>(ws);
    GroupBuffers g{};
    g.nb = (T + GT - 1) / GT;
    const size_t nb = g.nb;
    g.counts_blk = reinterpret_cast<int32_t*>(p); p += align256(nb * E * 4);
    g.masks_blk = reinterpret_cast<uint64_t*>(p); p += align256(nb * E * 8);
    g.blkoff = reinterpret_cast<int32_t*>(p); p += align256(nb * E * 4);
    g.err_blk = reinterpret_cast<int32_t*>(p); p += align256(nb * 4);
    g.scalars = reinterpret_cast<int32_t*>(p); p += align256(2 * 4);
    g.max_tiles = group_max_tiles(T, K, E);
    g.tiles = reinterpret_cast<int4*>(p); p += align256((size_t)g.max_tiles * 16);
    if (with_outputs) {
        g.counts = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * 4);
        g.offsets = reinterpret_cast<int32_t*>(p); p += align256((size_t)(E + 1) * 4);
        g.perm = reinterpret_cast<int32_t*>(p); p += align256((size_t)T * K * 4);
        g.uniq = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * 4);
    }
    return g;
}

size_t chunk_workspace_bytes(int T, int K, int E, int D, int F) {
    const size_t P = (size_t)T * K;
    return group_workspace_bytes(T, K, E, true) + align256(P * F * 2) + align256(P * D * 4);
}

ChunkWorkspace chunk_workspace_carve(void* ws, int T, int K, int E, int D, int F) {
    ChunkWorkspace c;
    c.g = group_workspace_carve(ws, T, K, E, true);
    const size_t P = (size_t)T * K;
    char* p = static_cast<char*>(ws) + group_workspace_bytes(T, K, E, true);
    c.h_bf16 = reinterpret_cast<uint16_t*>(p); p += align256(P * F * 2);
    c.ytk = reinterpret_cast<float*>(p);
    return c;
}

// ------------------------------------------------------------------------- launches
hipError_t launch_group(const int32_t* idx, int T, int K, int E, const GroupBuffers& g,
                        int32_t* n_unique_out, hipStream_t stream) {
    hipLaunchKernelGGL(group_count_kernel, dim3(g.nb), dim3(256), (size_t)E * 8, stream, idx, T, K, E,
                       g.counts_blk, reinterpret_cast<unsigned long long*>(g.masks_blk), g.err_blk);
    hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), (size_t)E * 4, stream, T, K, E, g.nb,
                       g.counts_blk, g.blkoff, g.err_blk, g.counts, g.offsets, g.uniq, g.tiles,
                       g.max_tiles, g.scalars, n_unique_out);
    hipLaunchKernelGGL(group_scatter_kernel, dim3(g.nb), dim3(256), 0, stream, idx, T, K, E,
                       reinterpret_cast<const unsigned long long*>(g.masks_blk), g.blkoff, g.offsets,
                       g.scalars, g.perm);
    return hipGetLastError();
}

hipError_t launch_chunk(const DevWeights& W, const uint16_t* x, int T, const int32_t* idx, const float* w,
                        int K, float* y, int32_t* n_unique_out, const ChunkWorkspace& ws,
                        hipStream_t stream) {
    hipError_t err = launch_group(idx, T, K, W.E, ws.g, n_unique_out, stream);
    if (err != hipSuccess) return err;

    GemmArgs gu{};
    gu.A = x;
    gu.perm = ws.g.perm;
    gu.K = K;
    gu.q0 = W.gate_q; gu.s0 = W.gate_s; gu.q1 = W.up_q; gu.s1 = W.up_s;
    gu.q0_stride = W.gate_q_stride; gu.s0_stride = W.gate_s_stride;
    gu.q1_stride = W.up_q_stride; gu.s1_stride = W.up_s_stride;
    gu.Kdim = W.D;
    gu.N = W.F;
    gu.tiles = ws.g.tiles;
    gu.scalars = ws.g.scalars;
    gu.nblk_n = (W.F + 4 * 32 - 1) / (4 * 32);
    gu.h_out = ws.h_bf16;
    const int max_items_gu = ws.g.max_tiles * gu.nblk_n;
    hipLaunchKernelGGL(gemm_kernel<GATEUP>, dim3(((max_items_gu + N_XCD - 1) / N_XCD) * N_XCD),
                       dim3(GEMM_THREADS), 0, stream, gu);

    GemmArgs dn{};
    dn.A = ws.h_bf16;
    dn.perm = ws.g.perm;
    dn.K = K;
    dn.q0 = W.down_q; dn.s0 = W.down_s;
    dn.q0_stride = W.down_q_stride; dn.s0_stride = W.down_s_stride;
    dn.Kdim = W.F;
    dn.N = W.D;
    dn.tiles = ws.g.tiles;
    dn.scalars = ws.g.scalars;
    dn.nblk_n = (W.D + 4 * 64 - 1) / (4 * 64);
    dn.y_out = ws.ytk;
    dn.wts = w;
    const int max_items_dn = ws.g.max_tiles * dn.nblk_n;
    hipLaunchKernelGGL(gemm_kernel<DOWN>, dim3(((max_items_dn + N_XCD - 1) / N_XCD) * N_XCD),
                       dim3(GEMM_THREADS), 0, stream, dn);

    const size_t n4 = (size_t)T * W.D / 4;
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, stream, ws.ytk, T, K, W.D,
                       ws.g.scalars, y);
    return hipGetLastError();
}

}  // namespace k3moe
