// dense.hip -- the LatentMoE block's dense products for a chunk of T >= 2 tokens,
// bf16 x bf16 with fp32 accumulation on v_mfma_f32_16x16x32_bf16.
//
// colibri PR #684, engine commit (Stable LatentMoE bullet): latent projections
// around the routed experts and two fused shared experts with SiTU-GLU.  A block
// runs three of these products:
//   x   = h Wdn^T                    [T, Dl] fp32
//   s   = SiTU(h Sg^T, h Su^T)       [T, Fs] bf16 (gate and up in one pass)
//   out = r Wup^T + s Sd^T           [T, Dh] fp32 (one reduction over two segments)
//
// Work item = (tile of MT token rows, tile of output columns, split of the
// reduction).  A workgroup of four waves stages its token rows in LDS, 64
// reduction columns per step (double buffer, 16-byte pieces swizzled by row);
// each wave streams its own two 16-row weight subtiles straight into MFMA B
// operands through a register ring NBB steps deep, so every weight byte is read
// by one wave of one workgroup per token tile.  At chunk sizes the weights
// dominate the traffic and there are few column tiles, so the reduction is split
// to fill the chip: each split writes its partial tile, counts itself on the
// tile's counter, and the last of the tile's splits sums the partials in split
// order (its own from registers) and applies the epilogue -- the same bits
// whichever split arrives last.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "device.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

using gemm::for_steps;
using gemm::lds_barrier;

constexpr int DKS = 64;           // reduction columns per step
constexpr int DROW = 2 * DKS;     // LDS bytes per staged row and step: 8 pieces of 16 bytes
constexpr int DWAVES = 4;
constexpr int DTHREADS = DWAVES * 64;
constexpr int DNBB = 4;           // weight ring depth (steps)
constexpr int DAS = 2;            // token-row register sets: rows are loaded DAS steps ahead
constexpr int DNSUB = 2;          // 16-row weight subtiles per wave (DENSE_SITU: half gate, half up)
constexpr int DMAXMS = 8;         // 16-row token subtiles per tile at most (registers)
constexpr int DCNT_STRIDE = 64;   // ints between counters (device-scope atomics on one line serialize)
constexpr double kCostFixed = 2.0, kCostPart = 8.0;  // split heuristic, in steps

// Output columns of a wave: DENSE_F32 one per weight row, DENSE_SITU one per gate/up row pair.
template <int EPI>
__host__ __device__ constexpr int wave_cols() { return EPI == DENSE_F32 ? 16 * DNSUB : 8 * DNSUB; }

// Partial floats of one work item: DWAVES waves x MS subtile rows x DNSUB x 4 x 64.
__host__ __device__ constexpr int item_floats(int ms) { return DWAVES * ms * DNSUB * 4 * 64; }

struct DenseArgs {
    const uint16_t* A[2];   // per segment: activations [T, K[s]] bf16, row-major
    const uint16_t* W[2];   // per segment: weights [N, K[s]] bf16 (DENSE_SITU: the gate half)
    const uint16_t* Wu;     // DENSE_SITU: the up half [N, K[0]]
    int K[2];               // per segment reduction length (multiple of 32; K[1] = 0: one segment)
    int nst0, nst;          // steps of segment 0, of both
    int T, N;
    int mtiles, ntiles, splits;
    float* outf;            // DENSE_F32: [T, N] fp32
    uint16_t* outb;         // DENSE_SITU: [T, N] bf16
    float* part;            // [tiles][splits] x item_floats(MS) partials (splits > 1)
    int32_t* cnt;           // [tiles] counters, DCNT_STRIDE apart, zero on entry (splits > 1)
};

// Slot of piece seg of staged row r: seg ^ dkey(r).  Two 128-byte rows share one
// 256-byte bank row; the 16 lanes of an A-fragment read take 16 consecutive rows
// at one segment, and this key gives the eight even rows eight distinct slots,
// and the eight odd rows too, so the 16 reads fall in 16 distinct bank groups.
__device__ __forceinline__ int dkey(int r) { return (r >> 1) & 7; }

// Two partial sums at once, past the XCD's own L2 (agent scope: other XCDs read them).
__device__ __forceinline__ void st_agent2(float* p, float a, float b) {
    const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent2(const float* p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
// every memory operation this wave issued so far has completed (stores included)
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Token-row pieces of one thread: piece c = (tid + i * DTHREADS) mod PIECES is row
// c / 8, segment c % 8 of a step (the segment is the same in every slot).  Rows
// past the tile re-read its last row; columns past the segment's K are stored as
// zeros.
template <int MT>
struct DPieces {
    static constexpr int PIECES = MT * 8;
    static constexpr int SLOTS = (PIECES + DTHREADS - 1) / DTHREADS;
    int seg;
    uint32_t arow[SLOTS];  // token row of each slot
    __device__ __forceinline__ static int row_of(int i) { return (((int)threadIdx.x + i * DTHREADS) % PIECES) >> 3; }
    __device__ __forceinline__ void init(int m0, int mrows) {
        seg = threadIdx.x & 7;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) arow[i] = (uint32_t)(m0 + min(row_of(i), mrows - 1));
    }
    __device__ __forceinline__ void load(const DenseArgs& a, uint4 (&v)[SLOTS], int g) const {
        const int s = g >= a.nst0 ? 1 : 0;
        const int K = a.K[s];
        const uint32_t c = (uint32_t)min((g - (s ? a.nst0 : 0)) * DKS + 8 * seg, K - 8);
        const uint16_t* A = a.A[s];
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) v[i] = *reinterpret_cast<const uint4*>(A + (arow[i] * (uint32_t)K + c));
    }
    __device__ __forceinline__ void store(const DenseArgs& a, const uint4 (&v)[SLOTS], uint8_t* buf, int g) const {
        const int s = g >= a.nst0 ? 1 : 0;
        const uint32_t m = (g - (s ? a.nst0 : 0)) * DKS + 8 * seg < a.K[s] ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int r = row_of(i);
            *reinterpret_cast<uint4*>(buf + r * DROW + 16 * (seg ^ dkey(r))) =
                make_uint4(v[i].x & m, v[i].y & m, v[i].z & m, v[i].w & m);
        }
    }
};

// One workgroup = one work item.  MS: 16-row subtiles of the token tile (MT = 16 MS).
template <int EPI, int MS>
__global__ __launch_bounds__(DTHREADS, 2) void dense_kernel(DenseArgs a) {
    constexpr int MT = 16 * MS;
    constexpr int BN = DWAVES * wave_cols<EPI>();
    constexpr int HALF = DNSUB / 2;
    __shared__ __attribute__((aligned(16))) uint8_t alds[2 * MT * DROW];
    __shared__ int s_last;

    // ---- work item (XCD-aware): the token tiles of one (column tile, split) are
    // consecutive, so they run on one XCD and share its L2 copy of the weights
    const int n_items = a.mtiles * a.ntiles * a.splits;
    const int item = gemm::xcd_item(n_items);
    if (item < 0) return;  // block-uniform
    const int mtile = item % a.mtiles;
    const int rest = item / a.mtiles;
    const int split = rest % a.splits, ntile = rest / a.splits;
    const int tile = ntile * a.mtiles + mtile;
    const int m0 = mtile * MT, mrows = min(MT, a.T - m0);
    const int g0 = (int)((long)split * a.nst / a.splits), g1 = (int)((long)(split + 1) * a.nst / a.splits);
    const int nloc = g1 - g0;  // >= 1 (splits <= steps)

    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N;
    // output columns of this wave from n0: DENSE_F32 subtile ns = rows n0 + 16 ns of
    // W; DENSE_SITU subtiles ns < HALF = gate rows n0 + 16 ns, the others the same
    // rows of up
    const int n0 = ntile * BN + wave * wave_cols<EPI>();

    // per segment and subtile: byte offset of this lane's weight row (clamped to N)
    uint32_t qoff[2][DNSUB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int ns = 0; ns < DNSUB; ++ns) {
            const int row = min(n0 + 16 * (EPI == DENSE_F32 ? ns : ns % HALF) + ln, N - 1);
            qoff[s][ns] = (uint32_t)row * (uint32_t)a.K[s] * 2u;
        }
    // the weights of step g (segment-local column 16 lg .. 16 lg + 15): two
    // 16-byte chunks per subtile; valid = inside the segment's K
    auto wload = [&](uint4 (&b)[DNSUB][2], bool& valid, int g) {
        const int s = g >= a.nst0 ? 1 : 0;
        const int K = a.K[s];
        const int col = (g - (s ? a.nst0 : 0)) * DKS + 16 * lg;
        valid = col < K;
        const uint32_t cb = 2u * (uint32_t)min(col, K - 16);
#pragma unroll
        for (int ns = 0; ns < DNSUB; ++ns) {
            const uint16_t* Wt = (EPI == DENSE_SITU && ns >= HALF) ? a.Wu : a.W[s];
            const char* p = reinterpret_cast<const char*>(Wt) + (qoff[s][ns] + cb);
            b[ns][0] = *reinterpret_cast<const uint4*>(p);
            b[ns][1] = *reinterpret_cast<const uint4*>(p + 16);
        }
    };

    DPieces<MT> ap;
    ap.init(m0, mrows);
    uint4 areg[DAS][DPieces<MT>::SLOTS];
    uint4 bring[DNBB][DNSUB][2];
    bool bvalid[DNBB];
#pragma unroll
    for (int u = 0; u < DNBB - 1; ++u) wload(bring[u], bvalid[u], g0 + min(u, nloc - 1));
#pragma unroll
    for (int u = 0; u < DAS; ++u) ap.load(a, areg[u], g0 + min(u, nloc - 1));
    ap.store(a, areg[0], alds, g0);
    __syncthreads();

    f32x4 acc[MS][DNSUB];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int ns = 0; ns < DNSUB; ++ns) acc[i][ns] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int akey = dkey(ln);  // key of fragment rows 16 i + ln

    // Per step t: load the rows of step t + DAS into the register set step t used and
    // the weights of step t + NBB - 1 into the ring slot step t - 1 used; compute
    // step t from LDS buffer t % 2 and ring slot t % NBB; store step t + 1's rows
    // into buffer (t + 1) % 2 (read last in step t - 1); barrier.
    // steps per loop body: a multiple of the ring depth, of the register sets and of
    // the two LDS buffers
    static_assert(DNBB % 2 == 0 && DAS % 2 == 0 && (DNBB % DAS == 0 || DAS % DNBB == 0), "loop body period");
    constexpr int PERIOD = DNBB > DAS ? DNBB : DAS;
    for_steps<PERIOD>(nloc, [&](auto uc, const int t) {
        constexpr int u = decltype(uc)::value;
        ap.load(a, areg[u % DAS], g0 + min(t + DAS, nloc - 1));
        wload(bring[(u + DNBB - 1) % DNBB], bvalid[(u + DNBB - 1) % DNBB], g0 + min(t + DNBB - 1, nloc - 1));
        const uint8_t* abuf = alds + (t & 1) * MT * DROW;
        const uint32_t vm = bvalid[u % DNBB] ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bf16x8 bop[DNSUB];
#pragma unroll
            for (int ns = 0; ns < DNSUB; ++ns) {
                const uint4 q = bring[u % DNBB][ns][j];
                bop[ns] = __builtin_bit_cast(bf16x8, make_uint4(q.x & vm, q.y & vm, q.z & vm, q.w & vm));
            }
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                const bf16x8 aop =
                    *reinterpret_cast<const bf16x8*>(abuf + (16 * i + ln) * DROW + 16 * ((2 * lg + j) ^ akey));
#pragma unroll
                for (int ns = 0; ns < DNSUB; ++ns)
                    acc[i][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[ns], acc[i][ns], 0, 0, 0);
            }
        }
        ap.store(a, areg[(u + 1) % DAS], alds + ((t + 1) & 1) * MT * DROW, g0 + min(t + 1, nloc - 1));
        lds_barrier();
    });

    // ---- split reduction: write the partial, count, the last split sums in order
    if (a.splits > 1) {
        float* pt = a.part + (size_t)tile * a.splits * item_floats(MS);
        float* mine = pt + (size_t)split * item_floats(MS) + (size_t)wave * (item_floats(MS) / DWAVES);
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
            for (int ns = 0; ns < DNSUB; ++ns)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    st_agent2(mine + (((i * DNSUB + ns) * 2 + h) * 64 + lane) * 2, acc[i][ns][2 * h],
                              acc[i][ns][2 * h + 1]);
        wait_memory();
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(a.cnt + (size_t)tile * DCNT_STRIDE, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == a.splits - 1;
        __syncthreads();
        if (!s_last) return;  // block-uniform
        f32x4 tot[MS][DNSUB];
        for (int sp = 0; sp < a.splits; ++sp) {  // split order, whichever split is last
            const float* ps = pt + (size_t)sp * item_floats(MS) + (size_t)wave * (item_floats(MS) / DWAVES);
#pragma unroll
            for (int i = 0; i < MS; ++i)
#pragma unroll
                for (int ns = 0; ns < DNSUB; ++ns) {
                    f32x4 v = acc[i][ns];
                    if (sp != split) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint64_t b = ld_agent2(ps + (((i * DNSUB + ns) * 2 + h) * 64 + lane) * 2);
                            v[2 * h] = __uint_as_float((uint32_t)b);
                            v[2 * h + 1] = __uint_as_float((uint32_t)(b >> 32));
                        }
                    }
                    if (sp == 0) {
                        tot[i][ns] = v;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) tot[i][ns][r] += v[r];
                    }
                }
        }
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
            for (int ns = 0; ns < DNSUB; ++ns) acc[i][ns] = tot[i][ns];
    }

    // ---- epilogue.  C layout: lane l, register r -> row 4 (l / 16) + r, column l % 16.
    if (n0 >= N) return;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m >= mrows) continue;
            const size_t row = (size_t)(m0 + m) * N;
            if constexpr (EPI == DENSE_F32) {
#pragma unroll
                for (int ns = 0; ns < DNSUB; ++ns)
                    if (n0 + 16 * ns < N) a.outf[row + n0 + 16 * ns + ln] = acc[i][ns][r];
            } else {
#pragma unroll
                for (int ns = 0; ns < HALF; ++ns)
                    if (n0 + 16 * ns < N)
                        a.outb[row + n0 + 16 * ns + ln] =
                            (uint16_t)f32_to_bf16_bits(situ_fast(acc[i][ns][r], acc[i][ns + HALF][r]));
            }
        }
}

__global__ __launch_bounds__(256) void dense_clear_kernel(int32_t* __restrict__ cnt, int n) {
    for (int i = (int)threadIdx.x; i < n; i += 256) cnt[(size_t)i * DCNT_STRIDE] = 0;
}

// 16-row subtiles of the token tile for T tokens.
int dense_ms(int T) { return std::min(DMAXMS, T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8); }

// Workgroups of dense_kernel<EPI, MS> the current device holds at once (CUs x
// resident workgroups per CU), cached per device and kernel.
template <int EPI, int MS>
int dense_slots() {
    static std::mutex mu;
    static int slots[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    std::lock_guard<std::mutex> lock(mu);
    if (slots[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dense_kernel<EPI, MS>, DTHREADS, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 2;
        slots[dev] = cus * per_cu;
    }
    return slots[dev];
}

template <int EPI, int MS>
hipError_t launch_dense_t(DenseArgs a, const DenseProblem& p, hipStream_t stream) {
    const DensePlan pl = dense_plan(p, dense_slots<EPI, MS>());
    a.mtiles = pl.mtiles;
    a.ntiles = pl.ntiles;
    a.splits = pl.splits;
    const long items = (long)a.mtiles * a.ntiles * a.splits;
    hipLaunchKernelGGL((dense_kernel<EPI, MS>), dim3(gemm::xcd_grid(items)), dim3(DTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_dense_ms(const DenseArgs& a, const DenseProblem& p, hipStream_t stream) {
    switch (dense_ms(p.T)) {
        case 1: return launch_dense_t<EPI, 1>(a, p, stream);
        case 2: return launch_dense_t<EPI, 2>(a, p, stream);
        case 4: return launch_dense_t<EPI, 4>(a, p, stream);
        default: return launch_dense_t<EPI, DMAXMS>(a, p, stream);
    }
}

}  // namespace

size_t dense_part_bytes(int T) {
    return (size_t)kDenseMaxSplitItems * item_floats(dense_ms(T)) * sizeof(float);
}

size_t dense_cnt_bytes() { return (size_t)kDenseMaxSplitItems * DCNT_STRIDE * sizeof(int32_t); }

DensePlan dense_plan(const DenseProblem& p, int slots) {
    DensePlan pl{};
    pl.ms = dense_ms(p.T);
    const int mt = 16 * pl.ms;
    pl.mtiles = (p.T + mt - 1) / mt;
    const int bn = DWAVES * (p.epi == DENSE_F32 ? wave_cols<DENSE_F32>() : wave_cols<DENSE_SITU>());
    pl.ntiles = (p.N + bn - 1) / bn;
    const int nst = (p.K[0] + DKS - 1) / DKS + (p.K[1] + DKS - 1) / DKS;
    const long tiles = (long)pl.mtiles * pl.ntiles;
    // splits: fewest rounds of resident workgroups per unit of reduction, with a
    // fixed cost per item (prologue, epilogue) and one for writing and summing a
    // partial; at least 4 steps per split
    pl.splits = 1;
    double best = 0.0;
    for (int s = 1; s <= kDenseMaxSplits && s <= std::max(1, nst / 4); ++s) {
        if (s > 1 && tiles * s > kDenseMaxSplitItems) break;
        const long rounds = (tiles * s + slots - 1) / slots;
        const double cost = (double)rounds * ((double)nst / s + kCostFixed + (s > 1 ? kCostPart * s : 0.0));
        if (s == 1 || cost < best) {
            best = cost;
            pl.splits = s;
        }
    }
    return pl;
}

hipError_t launch_dense_clear(int32_t* cnt, int ncnt_launches, hipStream_t stream) {
    hipLaunchKernelGGL(dense_clear_kernel, dim3(1), dim3(256), 0, stream, cnt, ncnt_launches * kDenseMaxSplitItems);
    return hipGetLastError();
}

hipError_t launch_dense(const DenseProblem& p, float* part, int32_t* cnt, hipStream_t stream) {
    if (p.T < 1 || p.N < 32 || p.N % 32 != 0 || p.K[0] < 32 || p.K[0] % 32 != 0 || p.K[1] < 0 || p.K[1] % 32 != 0 ||
        (p.epi == DENSE_SITU && (p.K[1] != 0 || p.Wu == nullptr)))
        return hipErrorInvalidValue;
    DenseArgs a{};
    a.A[0] = p.A[0]; a.A[1] = p.K[1] ? p.A[1] : p.A[0];
    a.W[0] = p.W[0]; a.W[1] = p.K[1] ? p.W[1] : p.W[0];
    a.Wu = p.Wu;
    a.K[0] = p.K[0]; a.K[1] = p.K[1] ? p.K[1] : p.K[0];
    a.nst0 = (p.K[0] + DKS - 1) / DKS;
    a.nst = a.nst0 + (p.K[1] + DKS - 1) / DKS;
    a.T = p.T; a.N = p.N;
    a.outf = p.outf; a.outb = p.outb;
    a.part = part; a.cnt = cnt;
    return p.epi == DENSE_F32 ? launch_dense_ms<DENSE_F32>(a, p, stream) : launch_dense_ms<DENSE_SITU>(a, p, stream);
}

}  // namespace k3moe
