// chunk.hip -- a chunk of tokens through the routed experts, expert union deduplicated.
//
// colibri PR #676, chunked-prefill paragraph: within a chunk the MoE loads each
// unique expert once and runs it for every position routed to it; PR #684,
// chunked-prefill commit: the position lists come from a counting sort.  On the
// GPU the union turns the per-token GEMVs into a grouped matrix product whose
// weight operand is each routed expert's MXFP4 bytes, streamed once per tile of
// up to 96 of its pairs (16 when the chunk is small).
//
// Kernels, in stream order (x arrives as fp32, or as bf16 through the bf16 entry):
//   group_count    per 64-token block: one 64-bit mask per expert (bit i = token
//                  t0+i chose it); popcounts are the block's per-expert counts
//   group_scan     one workgroup: per-expert totals, offsets, the union list,
//                  and the GEMM tile list (expert, first row, rows)
//   group_scatter  pair p = t*K+k goes to offsets[e] + (pairs of e in earlier
//                  blocks) + popcount(mask & bits below t): a stable counting sort
//   xsplit         (fp32 x) fp16(x); and x = hi + lo: hi = bf16(x), the exact
//                  residual lo as MXFP4 codes with one E8M0 scale per 32 (below)
//   gemm<GATEUP>   h = SiTU(x W_gate^T, x W_up^T) per tile (fp32 x: h in fp16)
//   gemm<DOWN>     y_pair = w_pair * (h W_down^T), fp32, at row p = t*K+k
//   combine        y_t = sum_k y_pair[t*K+k] in slot order
//
// GEMM structure (gfx950, v_mfma_f32_16x16x32_bf16, wave64):
//   workgroup = one (tile, column block): 8 waves at 96-row tiles (4 when the
//   weight scale rows of 8 would not fit in LDS), 4 waves two per CU at 16-row
//   tiles; each wave owns 32 (gate/up) or 64 (down) output columns.  The reduction runs in 128-column steps: the tile's A rows
//   (activations, shared by all waves) are loaded two steps ahead into registers
//   and stored into a double-buffered LDS tile, 16-byte pieces XOR-swizzled by
//   row; the weight operand never touches LDS: each lane loads 16 bytes (32
//   codes = one scale group) of one weight row into a register ring (2 steps
//   deep at 96-row tiles, 4 at 16-row tiles) and converts them with the gfx950
//   scaled fp4->bf16 converts straight into four MFMA B operands.  The k order inside a step is permuted (lane group g
//   owns columns 32g..32g+31, MFMA j takes 8j..8j+7 of them) identically for A
//   and B, which leaves the dot products unchanged.  Scale bytes of the
//   workgroup's weight rows are staged in LDS once.  Workgroup ids are remapped
//   so each XCD walks a contiguous run of (tile, column block) items: the column
//   blocks of one tile share that XCD's L2 copy of the tile's activations.
//
// fp32 activations.  A work item whose weights all decode to fp16 normals (every
// staged scale byte in 114..140: 0.5 * 2^(s-127) >= 2^-14, 6 * 2^(s-127) <= 65504)
// runs on v_mfma_f32_16x16x32_f16 with x and h rounded to fp16 (11 significant
// bits): the weights are exact in fp16, and the block output sits about 9e-4 from
// the exact one at the K3 shape (CPU emulation).  The test is per item, over the
// scale rows it stages anyway; an item that fails it (other scale bytes, byte 255,
// a ragged step, or some |x| past the fp16 range, flagged by the split) takes the
// bf16 path below, with h converted from fp16 to bf16 as its down item stages it.
//
// Rounding x to bf16 alone would move the block's output by
// about 7e-3 (rel-L2) on the K3-shape weights: where g = W_gate x sits in the
// SiTU-GLU's transition region, an error of 2^-9 |x| in every input shifts h by a
// large share of its range.  So x is split exactly, x = hi + lo with hi = bf16(x),
// and lo (|lo| <= 2^-9 |x|) enters as a second product: its codes are MXFP4 (e2m1
// with one E8M0 scale per 32 columns, chosen so the block's largest |lo| is at
// most 6 * 2^e, rounded to nearest even), multiplied with the weights' own FP4
// codes and scales by v_mfma_scale_f32_16x16x128_f8f6f4 into the same
// accumulators -- one MFMA per 128 columns against four bf16 MFMAs for hi.  The
// residual's own rounding is below 2^-11 of its block's largest value, i.e. about
// 2^-20 of x: the block output then sits about 1.5e-3 from the exact one, most of
// it the bf16 rounding of h.  The weights' scale byte 255 (which the scaled MFMA
// would read as NaN) is passed as 254 and the group's product added twice.
#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

using namespace gemm;

constexpr int GT = kGroupTokens;


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
        if (e == K3MOE_PRUNED) continue;  // a pruned slot is not a pair
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
                                                          int4* __restrict__ tiles, int max_tiles, int MT,
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
        scalars[2] = 0;  // raised by the x split when some |x| overflows fp16
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
        if (e == K3MOE_PRUNED) continue;
        const int ti = p / K - t0;
        const unsigned long long m = masks_blk[(size_t)b * E + e];
        const int rank = __popcll(m & ((1ull << ti) - 1ull));
        perm[offsets[e] + blkoff[(size_t)b * E + e] + rank] = p;
    }
}

// ----------------------------------------------------------------------------- GEMM
enum { GATEUP = 0, DOWN = 1 };

struct GemmArgs {
    const uint16_t* A;      // GATEUP: x bf16 [T, Kdim] by token (the high part for fp32 x);
                            // DOWN: h [P, Kdim] by grouped row (fp16 after an fp32-x gate/up, else bf16)
    const uint16_t* A16;    // GATEUP of fp32 x: x rounded to fp16 [T, Kdim]
    const uint8_t* alo;     // GATEUP with a low part: x - bf16(x) as FP4 codes [T, nsteps * 64]
    const uint8_t* alos;    //   and their E8M0 scales [T, nsteps * 4] (rows padded with zero codes)
    const int32_t* perm;    // grouped row -> pair id
    int K;                  // slots per token
    const uint8_t *q0, *s0, *q1, *s1;  // GATEUP: gate, up; DOWN: down (q1/s1 unused)
    int64_t q0_stride, s0_stride, q1_stride, s1_stride;
    int Kdim;               // reduction length (multiple of 32, <= 8192)
    int N;                  // output columns per expert (multiple of 32)
    const int4* tiles;
    const int32_t* scalars;  // [1] = number of tiles, [2] = some |x| overflows fp16
    int nblk_n;             // column blocks
    uint16_t* h_out;        // GATEUP output [P, N] (fp16 in the fp32-x kernels, else bf16), grouped rows
    float* y_out;           // DOWN output [P, N] fp32, pair rows
    const float* wts;       // DOWN: [P] routing weight of each pair
};

// GATEUP: a wave owns 32 columns of h and computes them from 16-row subtiles of
// the gate (n-subtiles 0, 1) and up (2, 3) weights.  DOWN: a wave owns 64 columns.
template <int MODE, int WAVES>
struct GemmShape {
    static constexpr int WN = (MODE == GATEUP) ? 32 : 64;     // output columns per wave
    static constexpr int BN = WAVES * WN;                     // output columns per workgroup
    static constexpr int TENSORS = (MODE == GATEUP) ? 2 : 1;  // weight tensors read
    static constexpr int SROWS = TENSORS * BN;                // weight rows whose scales sit in LDS
};


constexpr int LO_ROW = 64;  // bytes per staged low-part row and step: 128 FP4 codes

// A buffers, the row table, the low-part buffers and their per-step scale tables
// (with a low part), and the scale rows rounded up to whole 1 KiB copies.
inline size_t gemm_lds_bytes(int mt, int nb, int srows, int kdim, bool lo = false) {
    return (size_t)nb * mt * A_ROW + (size_t)mt * 8 + (lo ? (size_t)nb * mt * (LO_ROW + 4) : 0) +
           (((size_t)srows * (kdim / 32) + 1023) & ~(size_t)1023);
}




// A pieces of one loading thread (index lt of NT loading threads): piece
// c = (lt + i*NT) mod PIECES is tile row c/16, 16-byte segment c%16 of a step; it
// is stored at LDS slot seg ^ a_key(row) of the row, so the 16 lanes that read
// one MFMA fragment (16 rows, same segment) hit 16 different bank groups.
// Threads past the pieces repeat earlier ones (same bytes to the same place).
// Rows past the tile re-read its last row; columns past Kdim are clamped on load
// and stored as zeros.  NT is a multiple of 256, so a thread's segment and the
// row bits its swizzle key reads are the same for every i: per piece only the
// row's byte offset in A is kept (32 bits, added to the uniform base).
template <int MODE, int MT, int NT>
struct APieces {
    static_assert(NT % 256 == 0, "segment and key invariant over a thread's pieces");
    static constexpr int PIECES = MT * 16;
    static constexpr int SLOTS = (PIECES + NT - 1) / NT;
    uint32_t roff[SLOTS];  // byte offset of the piece's row in A
    int seg, key;          // the thread's segment, the key of its rows
    __device__ __forceinline__ static int row_of(int i) { return (((int)threadIdx.x + i * NT) % PIECES) >> 4; }
    __device__ __forceinline__ void init(const GemmArgs& a, int lt, int row0, int mrows) {
        seg = lt & 15;
        key = a_key(row_of(0));
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int rc = min(row_of(i), mrows - 1);
            const uint32_t row = (MODE == GATEUP) ? (uint32_t)(a.perm[row0 + rc] / a.K) : (uint32_t)(row0 + rc);
            roff[i] = row * (uint32_t)a.Kdim * 2u;
        }
    }
    // rows of A (16-bit elements, [rows, Kdim]) at the offsets computed by init
    __device__ __forceinline__ void load(const uint16_t* A, uint4 (&v)[SLOTS], int step, int Kdim) const {
        const uint32_t c = 2u * (uint32_t)min(step * KS + 8 * seg, Kdim - 8);
        const char* base = reinterpret_cast<const char*>(A);
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) v[i] = *reinterpret_cast<const uint4*>(base + (roff[i] + c));
    }
    // CVT: the loaded elements are fp16 and are stored as bf16 (round to nearest even)
    template <bool CVT = false>
    __device__ __forceinline__ void store(const uint4 (&v)[SLOTS], uint8_t* buf, int step, int Kdim) const {
        // mask word by word: a select between two uint4 objects would keep the
        // register arrays in memory
        const uint32_t m = step * KS + 8 * seg < Kdim ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            if constexpr (CVT) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const f16x2 hv = __builtin_bit_cast(f16x2, w[d]);
                    w[d] = f32_to_bf16_bits((float)hv[0]) | (f32_to_bf16_bits((float)hv[1]) << 16);
                }
            }
            *reinterpret_cast<uint4*>(buf + row_of(i) * A_ROW + 16 * (seg ^ key)) =
                make_uint4(w[0] & m, w[1] & m, w[2] & m, w[3] & m);
        }
    }
};


// Low-part pieces of one loading thread (index lt of NT): piece c = (lt + i*NT) mod
// PIECES is tile row c/4, 16-byte segment c%4 (32 codes = one scale group) of a
// step, stored at slot seg ^ ((row >> 2) & 3) of the row's 64 LDS bytes, so the 16
// lanes reading one fragment (16 rows, one segment) hit 16 distinct 16-byte slots
// of a 256-byte bank row.  Thread lt also carries the step's scale dword (four
// groups) of row lt % MT.  The low-part rows are padded to whole steps with zero
// codes, so no load is clamped or masked.
template <int MT, int NT>
struct LoPieces {
    static_assert(NT % 64 == 0, "segment and key invariant over a thread's pieces");
    static constexpr int PIECES = MT * 4;
    static constexpr int SLOTS = (PIECES + NT - 1) / NT;
    uint32_t roff[SLOTS];  // byte offset of the piece's row in the codes (plus its segment)
    uint32_t soff;         // byte offset of row lt % MT in the scales
    __device__ __forceinline__ static int row_of(int i) { return (((int)threadIdx.x + i * NT) % PIECES) >> 2; }
    __device__ __forceinline__ void init(const GemmArgs& a, int row0, int mrows, int nsteps) {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i)
            roff[i] = (uint32_t)(a.perm[row0 + min(row_of(i), mrows - 1)] / a.K) * (uint32_t)(nsteps * LO_ROW) +
                      16u * (threadIdx.x & 3);
        const int r = (int)threadIdx.x % MT;
        soff = (uint32_t)(a.perm[row0 + min(r, mrows - 1)] / a.K) * (uint32_t)(nsteps * 4);
    }
    __device__ __forceinline__ void load(const GemmArgs& a, u32x4 (&v)[SLOTS], uint32_t& sv, int step) const {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i)
            v[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.alo) + (roff[i] + step * LO_ROW));
        sv = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(a.alos) + (soff + 4 * step));
    }
    __device__ __forceinline__ void store(const u32x4 (&v)[SLOTS], uint32_t sv, uint8_t* buf, uint8_t* sbuf) const {
        const int seg = threadIdx.x & 3;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int r = row_of(i);
            *reinterpret_cast<u32x4*>(buf + r * LO_ROW + 16 * (seg ^ ((r >> 2) & 3))) = v[i];
        }
        *reinterpret_cast<uint32_t*>(sbuf + 4 * ((int)threadIdx.x % MT)) = sv;
    }
};

// Per-lane state of one work item that outlives the prologue: the activation
// pieces this thread stages (and with a low part, its pieces), the weight rows this
// lane streams, and the rings.
template <int MODE, int MT, int CW, int NBB, bool LO>
struct GemmState {
    using AP = APieces<MODE, MT, CW * 64>;
    using LP = LoPieces<MT, CW * 64>;
    static_assert(NBB >= 2 && NBB <= 4, "weight ring depth");
    // activation register sets: two (loads two steps ahead) for bf16 x; one (loads
    // one step ahead) with a low part, whose extra staging would not fit beside two
    static constexpr int AS = LO ? 1 : 2;
    AP ap;
    uint4 areg[AS][AP::SLOTS];
    LP lp;
    u32x4 lreg[AS][LO ? LP::SLOTS : 1];
    uint32_t lsreg[AS];
    uint32_t qoff[4];      // byte offset of this lane's weight row of subtile ns in its tensor
    uint32_t soff[4];      // byte offset of that row's scale bytes in the LDS scale region
    uint4 bring[NBB][4];
};

// Tensor of subtile ns (GATEUP: 0, 1 gate, 2, 3 up).
template <int MODE>
__device__ __forceinline__ constexpr int tensor_of(int ns) { return MODE == GATEUP ? (ns >> 1) : 0; }

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i fp4_operand(const uint4& q) {  // FP4: only the first four dwords are read
    return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}
__device__ __forceinline__ v8i fp4_operand(const u32x4& q) {
    return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

// The reduction of one work item after the prologue, with the number of 16-row
// subtiles (MS) fixed at compile time so the step body is straight-line code.
// EXACT adds the per-chunk s = 255 fix-up and the masking of weight columns past
// Kdim; the fast body is taken when no staged scale byte is 255 and Kdim is a
// multiple of 128.
//
// Per step t: load A(t + 2) into the register set A(t) used and the weights of
// step t + NBB - 1 into the ring slot step t - 1 used; read the scale bytes of
// step t + 1; compute step t from LDS buffer t % 2 and ring slot t % NBB; store
// A(t + 1) into buffer (t + 1) % 2 (read last in step t - 1); barrier.  All loads
// are ordinary vector loads, so the compiler's per-register waits stay exact
// across the loop.
//
// BODY: B_BF16 -- bf16 A and weights on v_mfma_f32_16x16x32_bf16 (plus the low
// part of x when the state has one); B_F16 -- fp16 A and weights on
// v_mfma_f32_16x16x32_f16 (every weight of the item an fp16 normal, no low part);
// B_CVT -- as B_BF16 with A loaded as fp16 and stored as bf16.  H16: the gate/up
// output h is stored as fp16 (else bf16).  asrc: the rows A is loaded from.
enum { B_BF16 = 0, B_F16 = 1, B_CVT = 2 };
// Launch kinds of the GEMM kernel (see launch_gemm).
enum { K_BF16 = 0, K_F16 = 1 };
template <int MODE, int MT, int CW, int NBB, bool LO, int MS, bool EXACT, int BODY, bool H16>
__device__ __forceinline__ void gemm_steps(const GemmArgs& a, GemmState<MODE, MT, CW, NBB, LO>& st, uint8_t* alds,
                                           uint8_t* llds, const uint8_t* slds, const char* qb0, const char* qb1,
                                           const int32_t* rperm, const float* rw, int row0, int mrows, int nb0,
                                           const uint16_t* asrc) {
    static_assert(!(EXACT && BODY == B_F16), "fp16 items are never exact");
    constexpr bool DO_LO = LO && BODY == B_BF16;  // the low part of x enters with the bf16 high part
    using SH = GemmShape<MODE, CW>;
    constexpr int WN = SH::WN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int akey = a_key(ln);  // swizzle key of this lane's fragment row (16 * i + ln)
    const int Kdim = a.Kdim, N = a.N, sb = Kdim >> 5;
    const int n0 = nb0 + wave * WN;
    const int nsteps = (Kdim + KS - 1) / KS;

    f32x4 acc[MS][4];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[i][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t scn[4];  // scale bytes of the next step
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) scn[ns] = slds[st.soff[ns] + min(lg, sb - 1)];

    // P steps per loop body: a multiple of the ring depth and of the two A register sets
    for_steps<(NBB % 2 == 0) ? NBB : 2 * NBB>(nsteps, [&](auto uc, const int step) {
        constexpr int u = decltype(uc)::value;
        constexpr int AS = GemmState<MODE, MT, CW, NBB, LO>::AS;
        if constexpr (AS == 2) st.ap.load(asrc, st.areg[u & 1], min(step + 2, nsteps - 1), Kdim);
        {
            const int col = min((step + NBB - 1) * KS + 32 * lg, Kdim - 32);
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
                st.bring[(u + NBB - 1) % NBB][ns] = *reinterpret_cast<const uint4*>(
                    (tensor_of<MODE>(ns) ? qb1 : qb0) + (st.qoff[ns] + (uint32_t)(col >> 1)));
        }
        uint32_t sc[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) sc[ns] = scn[ns];
        {
            const int nidx = min(4 * (step + 1) + lg, sb - 1);
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) scn[ns] = slds[st.soff[ns] + nidx];
        }
        const uint8_t* abuf = alds + (size_t)(u & 1) * MT * A_ROW;
        const bool valid = step * KS + 32 * lg < Kdim;
        float scf[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) scf[ns] = scale_operand(sc[ns]);
        if constexpr (DO_LO) {
            // the low part of x: FP4 x FP4 with both E8M0 scales, into the same
            // accumulators; the weight chunk is the B operand as loaded
            const uint8_t* lbuf = llds + (size_t)(u & 1) * MT * (LO_ROW + 4);
            const uint8_t* lsb = lbuf + MT * LO_ROW;
            const int lkey = (ln >> 2) & 3;
            int bsc[4];
            bool b255[4];
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
                b255[ns] = EXACT && sc[ns] == 255u;
                bsc[ns] = b255[ns] ? 254 : (int)sc[ns];
            }
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                const int r = 16 * i + ln;
                const u32x4 alo = *reinterpret_cast<const u32x4*>(lbuf + r * LO_ROW + 16 * (lg ^ lkey));
                const int sa = lsb[4 * r + lg];
                const v8i aop = fp4_operand(alo);
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) {
                    const v8i bop = fp4_operand(st.bring[u % NBB][ns]);
                    acc[i][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[i][ns], 4, 4, 0, sa,
                                                                                   0, bsc[ns]);
                    if constexpr (EXACT) {
                        // scale byte 255 = 2^128: the group at 2^127 once more
                        if (__any(b255[ns])) {
                            const v8i b2 = b255[ns] ? bop : v8i{0, 0, 0, 0, 0, 0, 0, 0};
                            acc[i][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, b2, acc[i][ns], 4, 4,
                                                                                           0, sa, 0, bsc[ns]);
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // the low part's fragments die before the converts
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (BODY == B_F16) {
                f16x8 bop[4];
#pragma unroll
                for (int ns = 0; ns < 4; ++ns)
                    bop[ns] = __builtin_bit_cast(f16x8, fp4x8_to_f16_nofix(pick(st.bring[u % NBB][ns], j), scf[ns]));
#pragma unroll
                for (int i = 0; i < MS; ++i) {
                    const f16x8 aop =
                        *reinterpret_cast<const f16x8*>(abuf + (16 * i + ln) * A_ROW + 16 * ((4 * lg + j) ^ akey));
#pragma unroll
                    for (int ns = 0; ns < 4; ++ns)
                        acc[i][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[ns], acc[i][ns], 0, 0, 0);
                }
            } else {
                bf16x8 bop[4];
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) {
                    if constexpr (EXACT)
                        bop[ns] = __builtin_bit_cast(bf16x8,
                                                     fp4x8_to_bf16(valid ? pick(st.bring[u % NBB][ns], j) : 0u, sc[ns]));
                    else
                        bop[ns] = __builtin_bit_cast(bf16x8, fp4x8_to_bf16_nofix(pick(st.bring[u % NBB][ns], j), scf[ns]));
                }
#pragma unroll
                for (int i = 0; i < MS; ++i) {
                    const bf16x8 aop =
                        *reinterpret_cast<const bf16x8*>(abuf + (16 * i + ln) * A_ROW + 16 * ((4 * lg + j) ^ akey));
#pragma unroll
                    for (int ns = 0; ns < 4; ++ns)
                        acc[i][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[ns], acc[i][ns], 0, 0, 0);
                }
            }
            // keep the scheduler from hoisting the next sub-step's operand reads
            // (registers for them would push the weight ring out of VGPRs)
            __builtin_amdgcn_sched_barrier(0);
        }
        st.ap.template store<BODY == B_CVT>(st.areg[(u + 1) % AS], alds + (size_t)((step + 1) & 1) * MT * A_ROW,
                                            step + 1, Kdim);
        if constexpr (DO_LO) {
            uint8_t* lb = llds + (size_t)((step + 1) & 1) * MT * (LO_ROW + 4);
            st.lp.store(st.lreg[0], st.lsreg[0], lb, lb + MT * LO_ROW);
        }
        if constexpr (AS == 1) {  // the next step's activations, one step ahead
            st.ap.load(asrc, st.areg[0], min(step + 2, nsteps - 1), Kdim);
            if constexpr (DO_LO) st.lp.load(a, st.lreg[0], st.lsreg[0], min(step + 2, nsteps - 1));
        }
        lds_barrier();
    });

    // epilogue.  C layout: lane l, register r -> row 4*(l/16)+r, column l%16.
    if (n0 >= N) return;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m >= mrows) continue;
            if (MODE == GATEUP) {
                uint16_t* hrow = a.h_out + (size_t)(row0 + m) * N;
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const float hv = situ_fast(acc[i][ns][r], acc[i][ns + 2][r]);
                    hrow[n0 + 16 * ns + ln] = H16 ? __builtin_bit_cast(uint16_t, (_Float16)hv)
                                                  : (uint16_t)f32_to_bf16_bits(hv);
                }
            } else {
                const int p = rperm[m];
                const float wp = rw[m];
                float* yrow = a.y_out + (size_t)p * N;
#pragma unroll
                for (int ns = 0; ns < 4; ++ns)
                    if (n0 + 16 * ns < N) yrow[n0 + 16 * ns + ln] = acc[i][ns][r] * wp;
            }
        }
    }
}

// Scale bytes whose e2m1 values are all fp16 normals: 0.5 * 2^(s-127) >= 2^-14 and
// 6 * 2^(s-127) <= 65504.
constexpr uint32_t kF16ScaleLo = 114, kF16ScaleHi = 140;

// Any staged scale byte equal to 255 among this thread's 16-byte pieces.
__device__ __forceinline__ int scales_have_255(const uint8_t* slds, int stotal, int nthreads) {
    int has = 0;
    for (int c = threadIdx.x; c < stotal; c += nthreads) {
        const uint4 v = *reinterpret_cast<const uint4*>(slds + 16 * c);
        const uint32_t w4[4] = {~v.x, ~v.y, ~v.z, ~v.w};  // 255 -> zero byte
#pragma unroll
        for (int d = 0; d < 4; ++d) has |= ((w4[d] - 0x01010101u) & ~w4[d] & 0x80808080u) != 0u;
    }
    return has;
}

// Any staged scale byte outside [lo, hi] among this thread's 16-byte pieces.
__device__ __forceinline__ int scales_outside(const uint8_t* slds, int stotal, int nthreads, uint32_t lo,
                                              uint32_t hi) {
    uint32_t bad = 0;
    for (int c = threadIdx.x; c < stotal; c += nthreads) {
        const uint4 v = *reinterpret_cast<const uint4*>(slds + 16 * c);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int b = 0; b < 4; ++b) bad |= (uint32_t)(((w4[d] >> (8 * b)) & 0xFFu) - lo > hi - lo);
    }
    return (int)bad;
}

// One workgroup = one (tile of <= MT pair rows of one expert, block of BN output
// columns), the whole reduction, in 128-column steps:
//   - each of CW waves streams the 16-byte weight chunks of its four 16-row
//     subtiles through an NBB-deep register ring and converts them in registers
//     into MFMA B operands;
//   - the tile's activation rows (shared by all waves) are loaded two steps
//     ahead into registers and stored into a double-buffered LDS tile, 16-byte
//     pieces XOR-swizzled by row; A fragments are read from there;
//   - one barrier per step; the scale bytes of the workgroup's weight rows are
//     copied to LDS up front, while the first activation and weight loads are
//     already in flight.
// Per-item setup shared by the kernel and the bf16 fallback of the fp32-x kernels:
// the staged rows' pair ids (item_init), the lane's weight rows and scale offsets
// and the first ring steps (item_ring).
template <int MODE, int MT, int CW, int NBB, bool LO>
__device__ __forceinline__ void item_init(const GemmArgs& a, GemmState<MODE, MT, CW, NBB, LO>& st, int row0,
                                          int mrows) {
    st.ap.init(a, threadIdx.x, row0, mrows);  // pair ids of the staged rows (first loads)
    if constexpr (LO) st.lp.init(a, row0, mrows, (a.Kdim + KS - 1) / KS);
}

template <int MODE, int MT, int CW, int NBB, bool LO>
__device__ __forceinline__ void item_ring(const GemmArgs& a, GemmState<MODE, MT, CW, NBB, LO>& st, int nb0,
                                          int srows_real, const char* qb0, const char* qb1) {
    using SH = GemmShape<MODE, CW>;
    const int lane = threadIdx.x & 63, ln = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Kdim = a.Kdim, N = a.N, sb = Kdim >> 5;
    const int n0 = nb0 + wave * SH::WN;
    const int nsteps = (Kdim + KS - 1) / KS;
    const uint32_t qrow = (uint32_t)Kdim >> 1;
    // ring entry ns: 16-row subtile ns (GATEUP: gate 0, 1, up 2, 3), lane row ln,
    // columns 32 * (lane / 16) of each step; rows clamped to real rows (columns
    // past N are computed from a repeated row and never stored)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const int r = (MODE == GATEUP) ? n0 + 16 * (ns & 1) + ln : n0 + 16 * ns + ln;
        const int row = min(r, N - 1);
        st.qoff[ns] = (uint32_t)row * qrow;
        st.soff[ns] = (uint32_t)(tensor_of<MODE>(ns) * srows_real * sb + (row - nb0) * sb);
    }
#pragma unroll
    for (int u = 0; u < NBB - 1; ++u) {
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int c0 = 32 * (lane >> 4);
            const int col = min(min(u, nsteps - 1) * KS + c0, Kdim - 32);
            st.bring[u][ns] = *reinterpret_cast<const uint4*>((tensor_of<MODE>(ns) ? qb1 : qb0) +
                                                              (st.qoff[ns] + (uint32_t)(col >> 1)));
        }
    }
}

// LDS of a work item: two A buffers, the row table, the low part's buffers (LO) and
// the weight scale rows.
template <int MT, bool LO>
struct ItemLds {
    uint8_t* alds;   // [2][MT][A_ROW]
    int32_t* rperm;  // [MT] pair of each tile row
    float* rw;       // [MT] its routing weight
    uint8_t* llds;   // LO: [2][MT * LO_ROW + MT * 4]
    uint8_t* slds;   // [TENSORS][rows][Kdim/32]
    __device__ __forceinline__ explicit ItemLds(uint8_t* smem) {
        alds = smem;
        rperm = reinterpret_cast<int32_t*>(smem + 2 * MT * A_ROW);
        rw = reinterpret_cast<float*>(rperm + MT);
        llds = reinterpret_cast<uint8_t*>(rw + MT);
        slds = llds + (LO ? 2 * MT * (LO_ROW + 4) : 0);
    }
};

// Run the staged item (scales and row table in LDS) on the bf16 MFMA: its first
// activation steps, the exact-path test, and the step body for its subtile count.
// BODY B_BF16 (x, with the low part when LO) or B_CVT (fp16 h staged as bf16); H16:
// h out in fp16.  Used by item_rest; the bf16 kernels write the same steps out.
template <int MODE, int MT, int CW, int NBB, bool LO, int BODY, bool H16>
__device__ __forceinline__ void item_bf16(const GemmArgs& a, GemmState<MODE, MT, CW, NBB, LO>& st,
                                          const ItemLds<MT, LO>& L, int row0, int mrows, int nb0, int stotal,
                                          const char* qb0, const char* qb1) {
    using ST = GemmState<MODE, MT, CW, NBB, LO>;
    constexpr int THREADS = CW * 64;
    const int Kdim = a.Kdim, nsteps = (Kdim + KS - 1) / KS;
    const int msub = min((mrows + 15) >> 4, MT / 16);
    st.ap.load(a.A, st.areg[0], 0, Kdim);
    if constexpr (ST::AS == 2) st.ap.load(a.A, st.areg[1], min(1, nsteps - 1), Kdim);
    if constexpr (LO) st.lp.load(a, st.lreg[0], st.lsreg[0], 0);
    st.ap.template store<BODY == B_CVT>(st.areg[0], L.alds, 0, Kdim);
    if constexpr (LO) st.lp.store(st.lreg[0], st.lsreg[0], L.llds, L.llds + MT * LO_ROW);
    if constexpr (ST::AS == 1) {  // step 1's activations into the one register set
        st.ap.load(a.A, st.areg[0], min(1, nsteps - 1), Kdim);
        if constexpr (LO) st.lp.load(a, st.lreg[0], st.lsreg[0], min(1, nsteps - 1));
    }
    __syncthreads();  // scales, the first A buffer and the row table are in LDS
    const bool exact = __syncthreads_or(scales_have_255(L.slds, stotal, THREADS)) != 0 || (Kdim % KS) != 0;
    if (exact) {
        gemm_steps<MODE, MT, CW, NBB, LO, MT / 16, true, BODY, H16>(a, st, L.alds, L.llds, L.slds, qb0, qb1, L.rperm,
                                                                    L.rw, row0, mrows, nb0, a.A);
        return;
    }
#define K3_TILE_CASE(MSV)                                                                                    \
    case MSV:                                                                                                \
        if constexpr (MSV <= MT / 16)                                                                        \
            gemm_steps<MODE, MT, CW, NBB, LO, MSV, false, BODY, H16>(a, st, L.alds, L.llds, L.slds, qb0, qb1, \
                                                                     L.rperm, L.rw, row0, mrows, nb0, a.A);  \
        break;
    switch (msub) {
        K3_TILE_CASE(1)
        K3_TILE_CASE(2)
        K3_TILE_CASE(3)
        K3_TILE_CASE(4)
        K3_TILE_CASE(5)
        K3_TILE_CASE(6)
        K3_TILE_CASE(7)
        K3_TILE_CASE(8)
        default: break;
    }
#undef K3_TILE_CASE
}

// The fp32-x kernels' items that the fp16 test rejected, on the bf16 MFMA with a
// state of their own.  Not inlined: its registers stay out of the fp16 path, and
// it redoes the per-item setup (the scales and the row table are already in LDS).
// The launch's GemmArgs is read where the kernel's arguments lie (the kernarg
// segment, whose first explicit argument sits at offset 0): handing the kernel
// parameter itself to a call would copy it to private memory in every workgroup.
template <int MODE, int MT, int CW, int NBB, bool LO>
__device__ __attribute__((noinline)) void item_rest(const void* kargs, int e, int row0, int mrows, int nb0,
                                                    int srows_real, int stotal) {
    const GemmArgs& a = *static_cast<const GemmArgs*>(kargs);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const ItemLds<MT, LO> L(smem);
    const char* qb0 = reinterpret_cast<const char*>(a.q0 + (size_t)e * a.q0_stride);
    const char* qb1 = (MODE == GATEUP) ? reinterpret_cast<const char*>(a.q1 + (size_t)e * a.q1_stride) : qb0;
    GemmState<MODE, MT, CW, NBB, LO> st;
    item_init(a, st, row0, mrows);
    item_ring(a, st, nb0, srows_real, qb0, qb1);
    item_bf16<MODE, MT, CW, NBB, LO, MODE == GATEUP ? B_BF16 : B_CVT, true>(a, st, L, row0, mrows, nb0, stotal, qb0,
                                                                           qb1);
}

// One workgroup = one (tile of <= MT pair rows of one expert, block of BN output
// columns), the whole reduction, in 128-column steps:
//   - each of CW waves streams the 16-byte weight chunks of its four 16-row
//     subtiles through an NBB-deep register ring and converts them in registers
//     into MFMA B operands;
//   - the tile's activation rows (shared by all waves) are loaded ahead into
//     registers and stored into a double-buffered LDS tile, 16-byte pieces
//     XOR-swizzled by row; A fragments are read from there;
//   - one barrier per step; the scale bytes of the workgroup's weight rows are
//     copied to LDS up front, while the first weight loads are already in flight.
// KIND K_BF16: bf16 x (with the low part when LO) and bf16 h.  K_F16 (fp32 x, and
// the down product after it): items whose weights are all fp16 normals run on the
// fp16 MFMA; the others go to item_rest.
template <int MODE, int MT, int CW, int NBB, bool LO, int KIND>
__global__ __launch_bounds__(CW * 64, (CW == 4 && MT == 16) ? 2 : 1) void gemm_kernel(GemmArgs a) {
    using SH = GemmShape<MODE, CW>;
    using ST = GemmState<MODE, MT, CW, NBB, LO>;
    constexpr int BN = SH::BN;
    constexpr int THREADS = CW * 64;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const ItemLds<MT, LO> L(smem);

    // ---- work item (XCD-aware): XCD x walks items [x*per, (x+1)*per)
    const int item = xcd_item(a.scalars[1] * a.nblk_n);
    if (item < 0) return;  // block-uniform
    const int tile = item / a.nblk_n, nblk = item % a.nblk_n;
    const int4 td = a.tiles[tile];
    const int e = td.x, row0 = td.y, mrows = td.z;  // 1 <= mrows <= MT
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Kdim = a.Kdim, N = a.N, sb = Kdim >> 5;
    const int nb0 = nblk * BN;
    const int nsteps = (Kdim + KS - 1) / KS;
    const int srows_real = min(BN, N - nb0);
    ST st;
    item_init(a, st, row0, mrows);

    // ---- scale bytes of the workgroup's rows: srows_real * sb contiguous bytes per
    // tensor (a multiple of 32, 16-byte aligned), copied global -> LDS directly
    // (global_load_lds) with tensor 1 right after tensor 0, so 16-byte piece c lands
    // at byte 16*c.  A wave whose 64 pieces all lie past the end skips the copy;
    // the lanes of the last wave that run past it re-copy the last piece into the
    // rounded-up tail of the region.
    const int spieces = (srows_real * sb) >> 4;
    const int stotal = SH::TENSORS * spieces;
    for (int c0 = 0; c0 < stotal; c0 += THREADS) {
        if (c0 + wave * 64 < stotal) {  // wave-uniform
            const int cc = min(c0 + tid, stotal - 1);
            const int tsel = cc >= spieces ? 1 : 0, pc = cc - tsel * spieces;
            const uint8_t* sbase = tsel == 0 ? a.s0 + (size_t)e * a.s0_stride : a.s1 + (size_t)e * a.s1_stride;
            __builtin_amdgcn_global_load_lds((glb_ptr_t)(sbase + (size_t)nb0 * sb + 16 * pc),
                                             (lds_ptr_t)(L.slds + 16 * (c0 + wave * 64)), 16, 0, 0);
        }
    }
    // the expert's weight tensors: wave-uniform bases, per-lane 32-bit row offsets
    const char* qb0 = reinterpret_cast<const char*>(a.q0 + (size_t)e * a.q0_stride);
    const char* qb1 = (MODE == GATEUP) ? reinterpret_cast<const char*>(a.q1 + (size_t)e * a.q1_stride) : qb0;
    item_ring(a, st, nb0, srows_real, qb0, qb1);  // first weight loads, behind the scale copy
    if (MODE == DOWN && tid < mrows) {  // pair id and routing weight of each tile row
        const int p = a.perm[row0 + tid];
        L.rperm[tid] = p;
        L.rw[tid] = a.wts[p];
    }

    if constexpr (KIND == K_BF16) {
        // bf16 activations: their first steps go out before the scale check (the
        // same steps as item_bf16, written out here: called, it costs spills)
        uint8_t* const alds = L.alds;
        uint8_t* const llds = L.llds;
        uint8_t* const slds = L.slds;
        const int msub = min((mrows + 15) >> 4, MT / 16);
        st.ap.load(a.A, st.areg[0], 0, Kdim);
        if constexpr (ST::AS == 2) st.ap.load(a.A, st.areg[1], min(1, nsteps - 1), Kdim);
        if constexpr (LO) st.lp.load(a, st.lreg[0], st.lsreg[0], 0);
        st.ap.store(st.areg[0], alds, 0, Kdim);
        if constexpr (LO) st.lp.store(st.lreg[0], st.lsreg[0], llds, llds + MT * LO_ROW);
        if constexpr (ST::AS == 1) {  // step 1's activations into the one register set
            st.ap.load(a.A, st.areg[0], min(1, nsteps - 1), Kdim);
            if constexpr (LO) st.lp.load(a, st.lreg[0], st.lsreg[0], min(1, nsteps - 1));
        }
        __syncthreads();  // scales, the first A buffer and the row table are in LDS
        const bool exact = __syncthreads_or(scales_have_255(slds, stotal, THREADS)) != 0 || (Kdim % KS) != 0;
        if (exact) {
            gemm_steps<MODE, MT, CW, NBB, LO, MT / 16, true, B_BF16, false>(a, st, alds, llds, slds, qb0, qb1, L.rperm,
                                                                           L.rw, row0, mrows, nb0, a.A);
            return;
        }
#define K3_TILE_CASE(MSV)                                                                                          \
    case MSV:                                                                                                      \
        if constexpr (MSV <= MT / 16)                                                                              \
            gemm_steps<MODE, MT, CW, NBB, LO, MSV, false, B_BF16, false>(a, st, alds, llds, slds, qb0, qb1, L.rperm, \
                                                                         L.rw, row0, mrows, nb0, a.A);             \
        break;
        switch (msub) {
            K3_TILE_CASE(1)
            K3_TILE_CASE(2)
            K3_TILE_CASE(3)
            K3_TILE_CASE(4)
            K3_TILE_CASE(5)
            K3_TILE_CASE(6)
            K3_TILE_CASE(7)
            K3_TILE_CASE(8)
            default: break;
        }
#undef K3_TILE_CASE
    } else {
        // the item runs on the fp16 MFMA when every weight it reads is an fp16
        // normal (scale bytes 114..140), no |x| overflows fp16 and the steps are whole
        __syncthreads();  // the scales and the row table are in LDS
        const bool f16 = __syncthreads_or(scales_outside(L.slds, stotal, THREADS, kF16ScaleLo, kF16ScaleHi)) == 0 &&
                         (Kdim % KS) == 0 && (MODE == DOWN || a.scalars[2] == 0);
        if (!f16) {  // block-uniform; the loads already made are dropped
            item_rest<MODE, MT, CW, NBB, LO>((const void*)__builtin_amdgcn_kernarg_segment_ptr(), e, row0, mrows,
                                             nb0, srows_real, stotal);
            return;
        }
        const uint16_t* src = MODE == GATEUP ? a.A16 : a.A;
        st.ap.load(src, st.areg[0], 0, Kdim);
        if constexpr (ST::AS == 2) st.ap.load(src, st.areg[1], min(1, nsteps - 1), Kdim);
        st.ap.store(st.areg[0], L.alds, 0, Kdim);
        if constexpr (ST::AS == 1) st.ap.load(src, st.areg[0], min(1, nsteps - 1), Kdim);
        __syncthreads();
        const int msub = min((mrows + 15) >> 4, MT / 16);
#define K3_TILE_CASE(MSV)                                                                                     \
    case MSV:                                                                                                 \
        if constexpr (MSV <= MT / 16)                                                                         \
            gemm_steps<MODE, MT, CW, NBB, LO, MSV, false, B_F16, true>(a, st, L.alds, L.llds, L.slds, qb0, qb1, \
                                                                       L.rperm, L.rw, row0, mrows, nb0, src); \
        break;
        switch (msub) {
            K3_TILE_CASE(1)
            K3_TILE_CASE(2)
            K3_TILE_CASE(3)
            K3_TILE_CASE(4)
            K3_TILE_CASE(5)
            K3_TILE_CASE(6)
            K3_TILE_CASE(7)
            K3_TILE_CASE(8)
            default: break;
        }
#undef K3_TILE_CASE
    }
}

template <int MODE, int MT, int CW, int NBB, bool LO, int KIND>
hipError_t launch_gemm_t(GemmArgs a, int max_tiles, hipStream_t stream) {
    using SH = GemmShape<MODE, CW>;
    a.nblk_n = (a.N + SH::BN - 1) / SH::BN;
    const size_t lds = gemm_lds_bytes(MT, 2, SH::SROWS, a.Kdim, LO);
    const long max_items = (long)max_tiles * a.nblk_n;
    const dim3 grid(xcd_grid(max_items));
    const void* fn = reinterpret_cast<const void*>(&gemm_kernel<MODE, MT, CW, NBB, LO, KIND>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_kernel<MODE, MT, CW, NBB, LO, KIND>), grid, dim3(CW * 64), lds, stream, a);
    return hipGetLastError();
}

// Two waves per SIMD.  16-row tiles: four waves, two workgroups per CU, a 4-deep
// weight ring.  96-row tiles (96 accumulator registers per lane): eight waves and a
// 2-deep ring, which is what fits two waves per SIMD beside two sets of activation
// registers.  LDS: two A buffers plus the staged scales; when the scales of eight
// waves' rows do not fit (long rows, e.g. a gate/up reduction of 8192), four waves
// with half the rows.
// KIND: K_BF16 (bf16 x and h), K_F16 (fp32 x and the fp16 h it produces: fp16 items
// where the weights allow, the rest on bf16).
template <int MODE, bool LO, int KIND>
hipError_t launch_gemm(const GemmArgs& a, int mt, int max_tiles, hipStream_t stream) {
    // 16-row tiles (experts with few pairs: weight-stream bound): 4-wave workgroups,
    // two per CU, so one workgroup's prologue and epilogue overlap the other's stream
    // (0.63 -> 0.58 ms for the 32-token chunk against one 8-wave workgroup per CU)
    if (mt == 16) return launch_gemm_t<MODE, 16, 4, 4, LO, KIND>(a, max_tiles, stream);
    if (gemm_lds_bytes(kTileRowsLarge, 2, GemmShape<MODE, 8>::SROWS, a.Kdim, LO) <= kLdsLimit)
        return launch_gemm_t<MODE, kTileRowsLarge, 8, 2, LO, KIND>(a, max_tiles, stream);
    return launch_gemm_t<MODE, kTileRowsLarge, 4, 2, LO, KIND>(a, max_tiles, stream);
}

// ------------------------------------------------------------------ x = hi + lo
// Eight lanes per 32-column group, four columns per lane: hi = bf16(x) (RNE); lo =
// x - hi exactly (0 where x or hi is not finite); the group's scale exponent e is
// the smallest with max|lo| <= 6 * 2^e (clamped to the E8M0 range), and each lo /
// 2^e is rounded to the nearest e2m1 value, ties to the even code.  Output rows of
// lo are padded to whole 128-column steps with zero codes (scale byte 127).
__device__ __forceinline__ uint32_t e2m1_rne(float v, float inv) {
    const float y = fabsf(v) * inv;  // <= 6 by the choice of the scale
    const uint32_t m = (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
                       (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) + (uint32_t)(y > 5.0f);
    return m | (v < 0.0f ? 8u : 0u);
}

// The same pass also writes x rounded to fp16 (RNE) for the fp16 items, and raises
// flag[0] when some finite |x| rounds past the fp16 range (>= 65520).
__global__ __launch_bounds__(256) void xsplit_kernel(const float* __restrict__ x, int T, int D,
                                                     uint16_t* __restrict__ xh, uint8_t* __restrict__ xl,
                                                     uint8_t* __restrict__ xls, uint16_t* __restrict__ x16,
                                                     int32_t* __restrict__ flag) {
    const int nsteps = (D + KS - 1) / KS, gpr = nsteps * 4;  // groups per padded row
    const size_t ngroups = (size_t)T * gpr;
    const int sub = threadIdx.x & 7;  // lane within the group
    const size_t stride = (size_t)gridDim.x * (blockDim.x / 8);
    // every lane of a group takes the same trip count (the loop bound is per group)
    for (size_t gi = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 8; gi < ngroups; gi += stride) {
        const size_t t = gi / gpr;
        const int g = (int)(gi % gpr);
        const bool real = 32 * g < D;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (real) {
            const float4 q = reinterpret_cast<const float4*>(x + t * D + 32 * g)[sub];
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        }
        uint32_t hb[4];
        float lo[4];
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hb[j] = f32_to_bf16_bits(v[j]);
            const float h = __uint_as_float(hb[j] << 16);
            lo[j] = (__builtin_isfinite(v[j]) && __builtin_isfinite(h)) ? v[j] - h : 0.0f;
            amax = max(amax, __float_as_uint(lo[j]) & 0x7FFFFFFFu);
        }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 8));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 8));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4, 8));
        int e = 0;
        if (amax >= 0x00800000u) {
            e = (int)(amax >> 23) - 127 - 2 + ((amax & 0x7FFFFFu) > 0x400000u ? 1 : 0);
            e = max(min(e, 127), -127);
        } else if (amax != 0u) {
            e = -127;
        }
        const float inv = __builtin_ldexpf(1.0f, -e);
        uint32_t codes = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) codes |= e2m1_rne(lo[j], inv) << (4 * j);
        if (real) {
            reinterpret_cast<uint2*>(xh + t * D + 32 * g)[sub] =
                make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            uint32_t f[4];
            bool over = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[j] = __builtin_bit_cast(uint16_t, (_Float16)v[j]);
                over |= __builtin_isfinite(v[j]) && fabsf(v[j]) >= 65520.0f;
            }
            reinterpret_cast<uint2*>(x16 + t * D + 32 * g)[sub] = make_uint2(f[0] | (f[1] << 16), f[2] | (f[3] << 16));
            if (over) flag[0] = 1;  // every writer stores the same value
        }
        reinterpret_cast<uint16_t*>(xl + t * (size_t)nsteps * LO_ROW + 16 * g)[sub] = (uint16_t)codes;
        if (sub == 0) xls[t * (size_t)gpr + g] = (uint8_t)(e + 127);
    }
}

// -------------------------------------------------------------------------- combine
// y_t = sum over slots in order of the weighted pair rows; pruned slots are skipped.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ytk, const int32_t* __restrict__ idx,
                                                      int T, int K, int D, const int32_t* __restrict__ scalars,
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
            // eight slots' loads in flight at once (every pair row exists, so the
            // loads need no branch); a pruned slot's row is read but not added
            for (int k0 = 0; k0 < K; k0 += 8) {
                float4 v[8];
                bool live[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = min(k0 + j, K - 1);
                    live[j] = k0 + j < K && idx[t * K + k] != K3MOE_PRUNED;
                    v[j] = reinterpret_cast<const float4*>(ytk + ((t * K + k) * (size_t)D))[dd];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (live[j]) {
                        acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w;
                    }
                }
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
    const int mt = tile_rows(T, K, E);
    return (int)((P + mt - 1) / mt + (E < P ? E : P));
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
    g.mt = tile_rows(T, K, E);
    g.tiles = reinterpret_cast<int4*>(p); p += align256((size_t)g.max_tiles * 16);
    if (with_outputs) {
        g.counts = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * 4);
        g.offsets = reinterpret_cast<int32_t*>(p); p += align256((size_t)(E + 1) * 4);
        g.perm = reinterpret_cast<int32_t*>(p); p += align256((size_t)T * K * 4);
        g.uniq = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * 4);
    }
    return g;
}

// group buffers, h [P, F] (16-bit), the pair rows [P, D] fp32, then (fp32 x) hi [T, D]
// bf16, the low part's codes [T, nsteps * 64] and scales [T, nsteps * 4], x in fp16 [T, D].
size_t chunk_workspace_bytes(int T, int K, int E, int D, int F) {
    const size_t P = (size_t)T * K, t = (size_t)T, ns = (size_t)(D + KS - 1) / KS;
    return group_workspace_bytes(T, K, E, true) + align256(P * F * 2) + align256(P * D * 4) +
           align256(t * D * 2) + align256(t * ns * LO_ROW) + align256(t * ns * 4) + align256(t * D * 2);
}

ChunkWorkspace chunk_workspace_carve(void* ws, int T, int K, int E, int D, int F) {
    ChunkWorkspace c;
    c.g = group_workspace_carve(ws, T, K, E, true);
    const size_t P = (size_t)T * K, t = (size_t)T, ns = (size_t)(D + KS - 1) / KS;
    char* p = static_cast<char*>(ws) + group_workspace_bytes(T, K, E, true);
    c.h_bf16 = reinterpret_cast<uint16_t*>(p); p += align256(P * F * 2);
    c.ytk = reinterpret_cast<float*>(p); p += align256(P * D * 4);
    c.x_hi = reinterpret_cast<uint16_t*>(p); p += align256(t * D * 2);
    c.x_lo = reinterpret_cast<uint8_t*>(p); p += align256(t * ns * LO_ROW);
    c.x_los = reinterpret_cast<uint8_t*>(p); p += align256(t * ns * 4);
    c.x16 = reinterpret_cast<uint16_t*>(p);
    return c;
}

// ------------------------------------------------------------------------- launches
hipError_t launch_group(const int32_t* idx, int T, int K, int E, const GroupBuffers& g,
                        int32_t* n_unique_out, hipStream_t stream) {
    hipLaunchKernelGGL(group_count_kernel, dim3(g.nb), dim3(256), (size_t)E * 8, stream, idx, T, K, E,
                       g.counts_blk, reinterpret_cast<unsigned long long*>(g.masks_blk), g.err_blk);
    hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), (size_t)E * 4, stream, T, K, E, g.nb,
                       g.counts_blk, g.blkoff, g.err_blk, g.counts, g.offsets, g.uniq, g.tiles,
                       g.max_tiles, g.mt, g.scalars, n_unique_out);
    hipLaunchKernelGGL(group_scatter_kernel, dim3(g.nb), dim3(256), 0, stream, idx, T, K, E,
                       reinterpret_cast<const unsigned long long*>(g.masks_blk), g.blkoff, g.offsets,
                       g.scalars, g.perm);
    return hipGetLastError();
}

hipError_t launch_chunk(const DevWeights& W, const float* x32, const uint16_t* xb16, int T, const int32_t* idx,
                        const float* w, int K, float* y, int32_t* n_unique_out, const ChunkWorkspace& ws,
                        hipStream_t stream) {
    hipError_t err = launch_group(idx, T, K, W.E, ws.g, n_unique_out, stream);
    if (err != hipSuccess) return err;
    const bool lo = x32 != nullptr;
    if (lo) {
        const size_t groups = (size_t)T * ((W.D + KS - 1) / KS) * 4;
        hipLaunchKernelGGL(xsplit_kernel, dim3(grid_for(groups, 256 / 8)), dim3(256), 0, stream, x32, T, W.D,
                           ws.x_hi, ws.x_lo, ws.x_los, ws.x16, ws.g.scalars + 2);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }

    GemmArgs gu{};
    gu.A = lo ? ws.x_hi : xb16;
    gu.A16 = ws.x16;
    gu.alo = ws.x_lo;
    gu.alos = ws.x_los;
    gu.perm = ws.g.perm;
    gu.K = K;
    gu.q0 = W.gate_q; gu.s0 = W.gate_s; gu.q1 = W.up_q; gu.s1 = W.up_s;
    gu.q0_stride = W.gate_q_stride; gu.s0_stride = W.gate_s_stride;
    gu.q1_stride = W.up_q_stride; gu.s1_stride = W.up_s_stride;
    gu.Kdim = W.D;
    gu.N = W.F;
    gu.tiles = ws.g.tiles;
    gu.scalars = ws.g.scalars;
    gu.h_out = ws.h_bf16;
    err = lo ? launch_gemm<GATEUP, true, K_F16>(gu, ws.g.mt, ws.g.max_tiles, stream)
             : launch_gemm<GATEUP, false, K_BF16>(gu, ws.g.mt, ws.g.max_tiles, stream);
    if (err != hipSuccess) return err;

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
    dn.y_out = ws.ytk;
    dn.wts = w;
    err = lo ? launch_gemm<DOWN, false, K_F16>(dn, ws.g.mt, ws.g.max_tiles, stream)   // h in fp16
             : launch_gemm<DOWN, false, K_BF16>(dn, ws.g.mt, ws.g.max_tiles, stream);
    if (err != hipSuccess) return err;

    return launch_combine(ws.ytk, idx, T, K, W.D, ws.g.scalars, y, stream);
}

hipError_t launch_combine(const float* ytk, const int32_t* idx, int T, int K, int D, const int32_t* scalars,
                          float* y, hipStream_t stream) {
    const size_t n4 = (size_t)T * D / 4;
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, stream, ytk, idx, T, K, D, scalars, y);
    return hipGetLastError();
}

}  // namespace k3moe
