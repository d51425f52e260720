// chunk_mx.hip -- the chunk path with MXFP8 activations and the MXFP4 weights
// consumed as stored by gfx950's scaled MFMA.
//
// The pages' fast CPU kernel quantizes activations in groups of 32 and takes the
// MXFP4 weights as they are (colibri PR #684, int8-activation commit); here the
// group of 32 stays, the activations become OCP MXFP8 (mx.hpp) in one or two
// parts, and the weights' e2m1 nibbles and ue8m0 bytes go straight into
// v_mfma_scale_f32_16x16x128_f8f6f4 as FP4 codes with their E8M0 block scales:
// no weight conversion at all, and one MFMA covers 128 reduction columns.  The
// weights keep their closed form for every scale byte: the MFMA would read E8M0
// 255 as NaN, so a work item whose staged scale rows hold a 255 runs a step body
// that passes 254 instead and adds those groups' products a second time
// (2^128 = 2 * 2^127, exact).
//
// Kernels, in stream order (x arrives as fp32):
//   group_*        as in the bf16 chunk path (chunk.hip)
//   mx_quant       x -> codes [parts][T][D], scales [parts][T][D/32]
//   gemm_mx<GATEUP> g, u over the quantized x, h = SiTU(g, u) in fp32, quantized
//                  to MXFP8 in the epilogue (the 32 columns of a block live in
//                  one 16-lane row: a DPP max gives the shared scale)
//   gemm_mx<DOWN>  y_pair = w_pair * (h W_down^T), fp32, at row p = t*K+k
//   combine        y_t = sum_k y_pair[t*K+k] in slot order
//
// GEMM structure: as in chunk.hip (one workgroup per (tile, column block), XCD-
// aware item order, weight chunks streamed through a register ring, activation
// rows staged two steps ahead through registers into a double-buffered LDS tile,
// one barrier per 128-column step), with these differences:
//   - a 16-byte weight chunk (32 codes of one scale group) is the B operand of
//     one lane as loaded: lane (col c, group g) holds columns 32g..32g+31 of a
//     step, which is the operand layout of the FP4 MFMA, and its scale operand is
//     that group's byte;
//   - the A operand of lane (row r, group g) is bytes 16g..16g+15 and 64+16g..
//     64+16g+15 of the row's 128 codes of the step, read from LDS as two 16-byte
//     pieces; its scale operand is the row's byte for group g;
//   - each step also stages the tile rows' four scale bytes per part (one dword
//     per row and part) into a small double-buffered LDS table.
// The reduction length must be a multiple of 128.
#include "device.hpp"
#include "gemm.hpp"
#include "launch.hpp"
#include "mx.hpp"

namespace k3moe {

namespace {

using namespace gemm;

typedef int v8i __attribute__((ext_vector_type(8)));

enum { MX_GATEUP = 0, MX_DOWN = 1 };

struct MxArgs {
    const uint8_t* aq;       // activation codes [parts][rows][Kdim]: GATEUP rows are tokens,
    const uint8_t* as;       //   DOWN rows grouped pairs; scales [parts][rows][Kdim/32]
    size_t aq_plane, as_plane;  // bytes from one part to the next
    const int32_t* perm;     // grouped row -> pair id
    int K;                   // slots per token
    const uint8_t *q0, *s0, *q1, *s1;  // GATEUP: gate, up; DOWN: down (q1/s1 unused)
    int64_t q0_stride, s0_stride, q1_stride, s1_stride;
    int Kdim;                // reduction length (multiple of 128, <= 8192)
    int N;                   // output columns per expert (multiple of 32)
    const int4* tiles;
    const int32_t* scalars;  // [1] = number of tiles
    int nblk_n;              // column blocks
    uint8_t* hq;             // GATEUP output codes [parts][P][N], grouped rows
    uint8_t* hs;             // GATEUP output scales [parts][P][N/32]
    size_t hq_plane, hs_plane;
    float* y_out;            // DOWN output [P, N] fp32, pair rows
    const float* wts;        // DOWN: [P] routing weight of each pair
};

template <int MODE, int WAVES>
struct MxShape {
    static constexpr int WN = (MODE == MX_GATEUP) ? 32 : 64;     // output columns per wave
    static constexpr int BN = WAVES * WN;                        // output columns per workgroup
    static constexpr int TENSORS = (MODE == MX_GATEUP) ? 2 : 1;  // weight tensors read
    static constexpr int SROWS = TENSORS * BN;                   // weight rows whose scales sit in LDS
};

// Two A buffers, two per-step scale tables, the row table, and the weight scale
// rows rounded up to whole 1 KiB copies.
inline size_t mx_lds_bytes(int mt, int parts, int srows, int kdim) {
    return (size_t)2 * mt * A_ROW + (size_t)2 * parts * mt * 4 + (size_t)mt * 8 +
           (((size_t)srows * (kdim / 32) + 1023) & ~(size_t)1023);
}

// Activation pieces of one loading thread (index lt of NT): piece c of a step is
// code bytes 16*(c%8)..+15 of part (c/8)%PARTS of tile row c/(8*PARTS), stored at
// 16-byte slot (part*8 + c%8) ^ (row%16) of the row's 256 LDS bytes, so the 16
// lanes reading one fragment (16 rows, same slot) hit 16 different bank groups.
// Thread lt also carries the step's scale dword of row r/PARTS, part r%PARTS,
// r = lt mod MT*PARTS.  Rows past the tile re-read its last row; threads past the
// pieces repeat earlier ones (same bytes to the same place).
template <int MODE, int MT, int NT, int PARTS>
struct MxPieces {
    static constexpr int PIECES = MT * 8 * PARTS;
    static constexpr int SLOTS = (PIECES + NT - 1) / NT;
    const uint8_t* src[SLOTS];
    int lds[SLOTS];
    const uint8_t* ssrc;  // scale row of this thread's (row, part)
    int slds;             // its byte offset in one scale table
    __device__ __forceinline__ void init(const MxArgs& a, int lt, int row0, int mrows) {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int c = (lt + i * NT) % PIECES;
            const int j = c & 7, q = c >> 3, pt = q % PARTS, r = q / PARTS;
            const int rc = min(r, mrows - 1);
            const size_t row = (MODE == MX_GATEUP) ? (size_t)(a.perm[row0 + rc] / a.K) : (size_t)(row0 + rc);
            src[i] = a.aq + pt * a.aq_plane + row * (size_t)a.Kdim + 16 * j;
            lds[i] = r * A_ROW + 16 * ((pt * 8 + j) ^ a_key(r));
        }
        {
            const int c = lt % (MT * PARTS);
            const int r = c / PARTS, pt = c % PARTS;
            const int rc = min(r, mrows - 1);
            const size_t row = (MODE == MX_GATEUP) ? (size_t)(a.perm[row0 + rc] / a.K) : (size_t)(row0 + rc);
            ssrc = a.as + pt * a.as_plane + row * (size_t)(a.Kdim / 32);
            slds = (pt * MT + r) * 4;
        }
    }
    __device__ __forceinline__ void load(u32x4 (&v)[SLOTS], uint32_t& sv, int step) const {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) v[i] = *reinterpret_cast<const u32x4*>(src[i] + step * KS);
        sv = *reinterpret_cast<const uint32_t*>(ssrc + 4 * step);
    }
    __device__ __forceinline__ void store(const u32x4 (&v)[SLOTS], uint32_t sv, uint8_t* buf, uint8_t* sbuf) const {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) *reinterpret_cast<u32x4*>(buf + lds[i]) = v[i];
        *reinterpret_cast<uint32_t*>(sbuf + slds) = sv;
    }
};

template <int MODE, int MT, int CW, int NBB, int PARTS>
struct MxState {
    using AP = MxPieces<MODE, MT, CW * 64, PARTS>;
    static_assert(NBB >= 2 && NBB <= 4, "weight ring depth");
    AP ap;
    u32x4 areg[2][AP::SLOTS];  // native vectors: a struct type here ends up in scratch
    uint32_t sreg[2];
    const uint8_t* bq[4];  // weight rows in HBM
    const uint8_t* bs[4];  // their scale rows in LDS
    u32x4 bring[NBB][4];
};

__device__ __forceinline__ v8i a_operand(const u32x4& lo, const u32x4& hi) {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
__device__ __forceinline__ v8i b_operand(const u32x4& q) {  // FP4: only the first four dwords are read
    return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

// Quantize the two values a lane holds of one 32-column block (columns ln and
// 16+ln of the block, the 16 lanes of a DPP row holding the rest) and store the
// codes and, from lane 0 of the row, the scale.  Returns the residuals.
__device__ __forceinline__ void mx_store_pair(float v0, float v1, int ln, uint8_t* qrow, uint8_t* srow, float& r0,
                                              float& r1) {
    const uint32_t amax = row16_max_u32(max(__float_as_uint(v0) & 0x7FFFFFFFu, __float_as_uint(v1) & 0x7FFFFFFFu));
    const uint32_t s = mx_scale_of(amax);
    uint32_t c0 = kE4M3NaN, c1 = kE4M3NaN;
    r0 = r1 = __builtin_nanf("");
    if (s != kMxNaNScale) {
        c0 = mx_encode(v0, s);
        c1 = mx_encode(v1, s);
        r0 = v0 - mx_decode(c0, s);
        r1 = v1 - mx_decode(c1, s);
    }
    qrow[ln] = (uint8_t)c0;
    qrow[16 + ln] = (uint8_t)c1;
    if (ln == 0) *srow = (uint8_t)s;
}

// The reduction of one work item after the prologue, MS 16-row subtiles.
// Per step t: load A(t + 2) (codes and scale dwords) into the register set A(t)
// used and the weights of step t + NBB - 1 into the ring slot step t - 1 used;
// read the weight scale bytes of step t + 1; compute step t from LDS buffer t % 2
// and ring slot t % NBB; store A(t + 1) into buffer (t + 1) % 2; barrier.
template <int MODE, int MT, int CW, int NBB, int PARTS, int MS, bool EXACT>
__device__ __forceinline__ void mx_steps(const MxArgs& a, MxState<MODE, MT, CW, NBB, PARTS>& st, uint8_t* alds,
                                         uint8_t* sl, const int32_t* rperm, const float* rw, int row0, int mrows,
                                         int nb0) {
    using SH = MxShape<MODE, CW>;
    constexpr int WN = SH::WN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int akey = a_key(ln);  // swizzle key of this lane's fragment row (16 * i + ln)
    const int Kdim = a.Kdim, N = a.N;
    const int n0 = nb0 + wave * WN;
    const int nsteps = Kdim / KS;

    f32x4 acc[MS][4];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[i][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t scn[4];  // weight scale bytes of the next step
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) scn[ns] = st.bs[ns][lg];

    // P steps per loop body: a multiple of the ring depth and of the two A register sets
    for_steps<(NBB % 2 == 0) ? NBB : 2 * NBB>(nsteps, [&](auto uc, const int step) {
        constexpr int u = decltype(uc)::value;
        st.ap.load(st.areg[u & 1], st.sreg[u & 1], min(step + 2, nsteps - 1));
        {
            const int col = min(step + NBB - 1, nsteps - 1) * KS + 32 * lg;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
                st.bring[(u + NBB - 1) % NBB][ns] = *reinterpret_cast<const u32x4*>(st.bq[ns] + (col >> 1));
        }
        uint32_t sc[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) sc[ns] = scn[ns];
        {
            const int nidx = 4 * min(step + 1, nsteps - 1) + lg;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) scn[ns] = st.bs[ns][nidx];
        }
        const uint8_t* abuf = alds + (size_t)(u & 1) * MT * A_ROW;
        const uint8_t* sbuf = sl + (size_t)(u & 1) * PARTS * MT * 4;
        int bsc[4];
        bool b255[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            b255[ns] = EXACT && sc[ns] == 255u;
            bsc[ns] = b255[ns] ? 254 : (int)sc[ns];
        }
        // A fragments in (part, subtile) order; the compiler interleaves the LDS
        // reads with the MFMAs (a scheduling barrier per fragment costs spills)
#pragma unroll
        for (int pt = 0; pt < PARTS; ++pt) {
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                const uint8_t* arow = abuf + (16 * i + ln) * A_ROW;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(arow + 16 * ((pt * 8 + lg) ^ akey));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(arow + 16 * ((pt * 8 + 4 + lg) ^ akey));
                const int sa = sbuf[(pt * MT + 16 * i + ln) * 4 + lg];
                const v8i aop = a_operand(lo, hi);
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) {
                    const v8i bop = b_operand(st.bring[u % NBB][ns]);
                    acc[i][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[i][ns], 0, 4, 0, sa,
                                                                                   0, bsc[ns]);
                    if constexpr (EXACT) {
                        // scale byte 255 = 2^128: the group at 2^127 once more
                        if (__any(b255[ns])) {
                            const v8i b2 = b255[ns] ? bop : v8i{0, 0, 0, 0, 0, 0, 0, 0};
                            acc[i][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, b2, acc[i][ns], 0, 4,
                                                                                           0, sa, 0, bsc[ns]);
                        }
                    }
                }
            }
        }
        st.ap.store(st.areg[(u + 1) & 1], st.sreg[(u + 1) & 1], alds + (size_t)((step + 1) & 1) * MT * A_ROW,
                    sl + (size_t)((step + 1) & 1) * PARTS * MT * 4);
        lds_barrier();
    });

    // epilogue.  C layout: lane l, register r -> row 4*(l/16)+r, column l%16.
    if (n0 >= N) return;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m >= mrows) continue;  // uniform over the 16 lanes of a DPP row
            if (MODE == MX_GATEUP) {
                const float h0 = situ_fast(acc[i][0][r], acc[i][2][r]);
                const float h1 = situ_fast(acc[i][1][r], acc[i][3][r]);
                const size_t hrow = (size_t)(row0 + m);
                float r0, r1;
                mx_store_pair(h0, h1, ln, a.hq + hrow * N + n0, a.hs + hrow * (N / 32) + n0 / 32, r0, r1);
                if (PARTS == 2)
                    mx_store_pair(r0, r1, ln, a.hq + a.hq_plane + hrow * N + n0,
                                  a.hs + a.hs_plane + hrow * (N / 32) + n0 / 32, r0, r1);
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

// One workgroup = one (tile of <= MT pair rows of one expert, block of BN output
// columns), the whole reduction.  Prologue: weight scale rows global -> LDS
// (global_load_lds), the lane's weight rows and the first ring steps, the first
// two activation steps, the DOWN row table; then the steps.
template <int MODE, int MT, int CW, int NBB, int PARTS>
__global__ __launch_bounds__(CW * 64, 1) void gemm_mx_kernel(MxArgs a) {
    using SH = MxShape<MODE, CW>;
    using ST = MxState<MODE, MT, CW, NBB, PARTS>;
    constexpr int BN = SH::BN, WN = SH::WN;
    constexpr int THREADS = CW * 64;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* alds = smem;                                          // [2][MT][A_ROW]
    uint8_t* sl = smem + 2 * MT * A_ROW;                           // [2][PARTS][MT] dwords
    int32_t* rperm = reinterpret_cast<int32_t*>(sl + 2 * PARTS * MT * 4);  // [MT]
    float* rw = reinterpret_cast<float*>(rperm + MT);                       // [MT]
    uint8_t* slds = reinterpret_cast<uint8_t*>(rw + MT);                    // [TENSORS][rows][Kdim/32]

    const int item = xcd_item(a.scalars[1] * a.nblk_n);
    if (item < 0) return;  // block-uniform
    const int tile = item / a.nblk_n, nblk = item % a.nblk_n;
    const int4 td = a.tiles[tile];
    const int e = td.x, row0 = td.y, mrows = td.z;  // 1 <= mrows <= MT
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15;
    const int Kdim = a.Kdim, N = a.N, sb = Kdim >> 5;
    const int nb0 = nblk * BN;
    const int n0 = nb0 + wave * WN;
    const int nsteps = Kdim / KS;

    ST st;
    st.ap.init(a, tid, row0, mrows);

    // weight scale rows: srows_real * sb contiguous bytes per tensor (sb is a
    // multiple of 4 and srows_real of 32, so a multiple of 16 bytes), tensor 1
    // right after tensor 0
    const int srows_real = min(BN, N - nb0);
    const int spieces = (srows_real * sb) >> 4;
    const int stotal = SH::TENSORS * spieces;
    for (int c0 = 0; c0 < stotal; c0 += THREADS) {
        if (c0 + wave * 64 < stotal) {  // wave-uniform
            const int cc = min(c0 + tid, stotal - 1);
            const int tsel = cc >= spieces ? 1 : 0, pc = cc - tsel * spieces;
            const uint8_t* sbase = tsel == 0 ? a.s0 + (size_t)e * a.s0_stride : a.s1 + (size_t)e * a.s1_stride;
            __builtin_amdgcn_global_load_lds((glb_ptr_t)(sbase + (size_t)nb0 * sb + 16 * pc),
                                             (lds_ptr_t)(slds + 16 * (c0 + wave * 64)), 16, 0, 0);
        }
    }

    const size_t qrow = (size_t)Kdim >> 1;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const int tsel = (MODE == MX_GATEUP) ? (ns >> 1) : 0;
        const int r = (MODE == MX_GATEUP) ? n0 + 16 * (ns & 1) + ln : n0 + 16 * ns + ln;
        const int row = min(r, N - 1);
        const uint8_t* q = (tsel == 0) ? a.q0 + (size_t)e * a.q0_stride : a.q1 + (size_t)e * a.q1_stride;
        st.bq[ns] = q + (size_t)row * qrow;
        st.bs[ns] = slds + (size_t)tsel * srows_real * sb + (size_t)(row - nb0) * sb;
    }
    {
        const int lg = lane >> 4;
#pragma unroll
        for (int u = 0; u < NBB - 1; ++u) {
            const int col = min(u, nsteps - 1) * KS + 32 * lg;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) st.bring[u][ns] = *reinterpret_cast<const u32x4*>(st.bq[ns] + (col >> 1));
        }
    }
    st.ap.load(st.areg[0], st.sreg[0], 0);
    st.ap.load(st.areg[1], st.sreg[1], min(1, nsteps - 1));
    if (MODE == MX_DOWN && tid < mrows) {
        const int p = a.perm[row0 + tid];
        rperm[tid] = p;
        rw[tid] = a.wts[p];
    }
    st.ap.store(st.areg[0], st.sreg[0], alds, sl);
    __syncthreads();  // weight scales, the first A buffer and the row table are in LDS

    // any weight scale byte equal to 255 in the staged rows?
    int has255 = 0;
    for (int c = tid; c < stotal; c += THREADS) {
        const uint4 v = *reinterpret_cast<const uint4*>(slds + 16 * c);
        const uint32_t w4[4] = {~v.x, ~v.y, ~v.z, ~v.w};  // 255 -> zero byte
#pragma unroll
        for (int d = 0; d < 4; ++d) has255 |= ((w4[d] - 0x01010101u) & ~w4[d] & 0x80808080u) != 0u;
    }
    if (__syncthreads_or(has255) != 0) {
        mx_steps<MODE, MT, CW, NBB, PARTS, MT / 16, true>(a, st, alds, sl, rperm, rw, row0, mrows, nb0);
        return;
    }

    const int msub = min((mrows + 15) >> 4, MT / 16);
#define K3_MX_CASE(MSV)                                                                          \
    case MSV:                                                                                    \
        if constexpr (MSV <= MT / 16)                                                            \
            mx_steps<MODE, MT, CW, NBB, PARTS, MSV, false>(a, st, alds, sl, rperm, rw, row0, mrows, nb0); \
        break;
    switch (msub) {
        K3_MX_CASE(1)
        K3_MX_CASE(2)
        K3_MX_CASE(3)
        K3_MX_CASE(4)
        K3_MX_CASE(5)
        K3_MX_CASE(6)
        K3_MX_CASE(7)
        K3_MX_CASE(8)
        default: break;
    }
#undef K3_MX_CASE
}

template <int MODE, int MT, int CW, int NBB, int PARTS>
hipError_t launch_mx_t(MxArgs a, int max_tiles, hipStream_t stream) {
    using SH = MxShape<MODE, CW>;
    a.nblk_n = (a.N + SH::BN - 1) / SH::BN;
    const size_t lds = mx_lds_bytes(MT, PARTS, SH::SROWS, a.Kdim);
    const dim3 grid(xcd_grid((long)max_tiles * a.nblk_n));
    const void* fn = reinterpret_cast<const void*>(&gemm_mx_kernel<MODE, MT, CW, NBB, PARTS>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_mx_kernel<MODE, MT, CW, NBB, PARTS>), grid, dim3(CW * 64), lds, stream, a);
    return hipGetLastError();
}

// Tile and ring shapes as in the bf16 path: 16-row tiles with a 4-deep ring,
// large tiles with a 2-deep ring, four waves when eight waves' scale rows do not
// fit in LDS.
template <int MODE, int PARTS>
hipError_t launch_mx_parts(const MxArgs& a, int mt, int max_tiles, hipStream_t stream) {
    if (mt == 16) return launch_mx_t<MODE, 16, 8, 4, PARTS>(a, max_tiles, stream);
    if (mx_lds_bytes(kTileRowsLarge, PARTS, MxShape<MODE, 8>::SROWS, a.Kdim) <= kLdsLimit)
        return launch_mx_t<MODE, kTileRowsLarge, 8, 2, PARTS>(a, max_tiles, stream);
    return launch_mx_t<MODE, kTileRowsLarge, 4, 2, PARTS>(a, max_tiles, stream);
}

template <int MODE>
hipError_t launch_mx(const MxArgs& a, int parts, int mt, int max_tiles, hipStream_t stream) {
    return parts == 2 ? launch_mx_parts<MODE, 2>(a, mt, max_tiles, stream)
                      : launch_mx_parts<MODE, 1>(a, mt, max_tiles, stream);
}

// ---------------------------------------------------------------- quantization
// One thread per 32-value block: fp32 or bf16 in, PARTS code planes and scale
// planes out.
template <typename IN, int PARTS>
__global__ __launch_bounds__(256) void mx_quant_kernel(const IN* __restrict__ v, size_t nblk,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       size_t code_plane, size_t scale_plane) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        float x[32];
        if constexpr (sizeof(IN) == 2) {
            const uint4* src = reinterpret_cast<const uint4*>(v + 32 * b);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 w = src[q];
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[8 * q + 2 * j] = __uint_as_float(ws[j] << 16);
                    x[8 * q + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
                }
            }
        } else {
            const float4* src = reinterpret_cast<const float4*>(v + 32 * b);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 w = src[q];
                x[4 * q] = w.x; x[4 * q + 1] = w.y; x[4 * q + 2] = w.z; x[4 * q + 3] = w.w;
            }
        }
#pragma unroll
        for (int pt = 0; pt < PARTS; ++pt) {
            uint32_t amax = 0;
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = max(amax, __float_as_uint(x[j]) & 0x7FFFFFFFu);
            const uint32_t s = mx_scale_of(amax);
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float xv = x[4 * q + j];
                    uint32_t c = kE4M3NaN;
                    float res = __builtin_nanf("");
                    if (s != kMxNaNScale) {
                        c = mx_encode(xv, s);
                        res = xv - mx_decode(c, s);
                    }
                    packed |= c << (8 * j);
                    x[4 * q + j] = res;  // the next part quantizes the residual
                }
                w[q] = packed;
            }
            uint4* dst = reinterpret_cast<uint4*>(codes + pt * code_plane + 32 * b);
            dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            scales[pt * scale_plane + b] = (uint8_t)s;
        }
    }
}

int grid_blocks(size_t n, int per_block) {
    size_t b = (n + per_block - 1) / per_block;
    return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

hipError_t launch_mx_quant(const void* v, bool bf16, size_t n, int parts, uint8_t* codes, uint8_t* scales,
                           size_t code_plane, size_t scale_plane, hipStream_t stream) {
    const size_t nblk = n / 32;
    const dim3 grid(grid_blocks(nblk, 256)), block(256);
    if (bf16) {
        if (parts == 2)
            hipLaunchKernelGGL((mx_quant_kernel<uint16_t, 2>), grid, block, 0, stream,
                               static_cast<const uint16_t*>(v), nblk, codes, scales, code_plane, scale_plane);
        else
            hipLaunchKernelGGL((mx_quant_kernel<uint16_t, 1>), grid, block, 0, stream,
                               static_cast<const uint16_t*>(v), nblk, codes, scales, code_plane, scale_plane);
    } else {
        if (parts == 2)
            hipLaunchKernelGGL((mx_quant_kernel<float, 2>), grid, block, 0, stream, static_cast<const float*>(v),
                               nblk, codes, scales, code_plane, scale_plane);
        else
            hipLaunchKernelGGL((mx_quant_kernel<float, 1>), grid, block, 0, stream, static_cast<const float*>(v),
                               nblk, codes, scales, code_plane, scale_plane);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ workspace
// group buffers, then x codes [2][T][D] and scales [2][T][D/32], h codes [2][P][F]
// and scales [2][P][F/32], pair outputs [P][D] fp32 (planes sized for two parts).
size_t chunk_mx_workspace_bytes(int T, int K, int E, int D, int F) {
    const size_t P = (size_t)T * K;
    return group_workspace_bytes(T, K, E, true) + align256(2 * (size_t)T * D) + align256(2 * (size_t)T * D / 32) +
           align256(2 * P * F) + align256(2 * P * F / 32) + align256(P * D * 4);
}

ChunkMxWorkspace chunk_mx_workspace_carve(void* ws, int T, int K, int E, int D, int F) {
    ChunkMxWorkspace c;
    c.g = group_workspace_carve(ws, T, K, E, true);
    const size_t P = (size_t)T * K;
    char* p = static_cast<char*>(ws) + group_workspace_bytes(T, K, E, true);
    c.xq = reinterpret_cast<uint8_t*>(p); p += align256(2 * (size_t)T * D);
    c.xs = reinterpret_cast<uint8_t*>(p); p += align256(2 * (size_t)T * D / 32);
    c.hq = reinterpret_cast<uint8_t*>(p); p += align256(2 * P * F);
    c.hs = reinterpret_cast<uint8_t*>(p); p += align256(2 * P * F / 32);
    c.ytk = reinterpret_cast<float*>(p);
    return c;
}

hipError_t launch_chunk_mx(const DevWeights& W, const float* x, int T, const int32_t* idx, const float* w,
                           int K, int parts, float* y, int32_t* n_unique_out, const ChunkMxWorkspace& ws,
                           hipStream_t stream) {
    hipError_t err = launch_group(idx, T, K, W.E, ws.g, n_unique_out, stream);
    if (err != hipSuccess) return err;
    const size_t P = (size_t)T * K;
    const size_t xplane = (size_t)T * W.D, xsplane = xplane / 32;
    err = launch_mx_quant(x, false, (size_t)T * W.D, parts, ws.xq, ws.xs, xplane, xsplane, stream);
    if (err != hipSuccess) return err;

    MxArgs gu{};
    gu.aq = ws.xq; gu.as = ws.xs; gu.aq_plane = xplane; gu.as_plane = xsplane;
    gu.perm = ws.g.perm;
    gu.K = K;
    gu.q0 = W.gate_q; gu.s0 = W.gate_s; gu.q1 = W.up_q; gu.s1 = W.up_s;
    gu.q0_stride = W.gate_q_stride; gu.s0_stride = W.gate_s_stride;
    gu.q1_stride = W.up_q_stride; gu.s1_stride = W.up_s_stride;
    gu.Kdim = W.D;
    gu.N = W.F;
    gu.tiles = ws.g.tiles;
    gu.scalars = ws.g.scalars;
    gu.hq = ws.hq; gu.hs = ws.hs; gu.hq_plane = P * W.F; gu.hs_plane = P * W.F / 32;
    err = launch_mx<MX_GATEUP>(gu, parts, ws.g.mt, ws.g.max_tiles, stream);
    if (err != hipSuccess) return err;

    MxArgs dn{};
    dn.aq = ws.hq; dn.as = ws.hs; dn.aq_plane = P * W.F; dn.as_plane = P * W.F / 32;
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
    err = launch_mx<MX_DOWN>(dn, parts, ws.g.mt, ws.g.max_tiles, stream);
    if (err != hipSuccess) return err;
    return launch_combine(ws.ytk, idx, T, K, W.D, ws.g.scalars, y, stream);
}

}  // namespace k3moe
