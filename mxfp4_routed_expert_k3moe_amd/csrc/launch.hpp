// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "k3moe.h"  // status codes, limits and the pruned-slot marker shared with the kernels

namespace k3moe {

// Expert weights as the kernels see them (plain values, passed by value).
struct DevWeights {
    int32_t E, D, F;
    const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
    int64_t gate_q_stride, gate_s_stride, up_q_stride, up_s_stride, down_q_stride, down_s_stride;
};

// ------------------------------------------------------------------ route
hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, double top_p, int32_t* idx,
                        float* w, int32_t* n_kept, hipStream_t stream);

// ------------------------------------------------------------------ decode
constexpr int kDecodeWaves = 4;  // gate/up waves per workgroup (16 weight rows each)

struct DecodeWorkspace {
    float* h;      // [K, F]  SiTU-GLU outputs per slot
    float* ypart;  // [K, D]  down-projection outputs per slot
    int32_t* cnt;  // counters of the down kernel's folded combine (cleared by gate/up)
};
size_t decode_workspace_bytes(int K, int D, int F);
// Address of the current device's fixed scratch array (K3MOE_NOALLOC_SCRATCH_BYTES),
// looked up once per device; allocates nothing.
hipError_t noalloc_scratch(void** out);
DecodeWorkspace decode_workspace_carve(void* ws, int K, int D, int F);
// With both events given, the gate/up kernel is launched through
// hipExtLaunchKernelGGL, which records ev_start as it starts and ev_stop as it ends.
hipError_t launch_decode(const DevWeights& W, const float* x, const int32_t* idx, const float* w, int K,
                         float* y, const DecodeWorkspace& ws, hipStream_t stream, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);
// With both events given, the kernel is launched through hipExtLaunchKernelGGL,
// which records ev_start as the kernel starts and ev_stop as it ends.  split: -1
// serves the kept slots with 32-row split workgroups when idx holds a pruned slot,
// 0 never, 1 always (a caller that launches a token's slots in parts passes the
// token's own choice, so every part sums in the token's order).
hipError_t launch_decode_gateup(const DevWeights& W, const float* x, const int32_t* idx, int K, float* h,
                                hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                                int split = -1, int32_t* cnt = nullptr);
// cnt (from the same call's gate/up launch, which cleared it): the combine is folded
// into the down kernel; nullptr: a separate combine kernel.
hipError_t launch_decode_down(const DevWeights& W, const float* h, const int32_t* idx, const float* w, int K,
                              float* ypart, float* y, hipStream_t stream, int32_t* cnt = nullptr);

// ------------------------------------------------------------------ chunk
constexpr int kGroupTokens = 64;   // tokens per grouping block (one u64 mask bit each)
// GEMM tile height (pairs of one expert per tile): 16 when experts average at most
// 16 pairs, else kTileRowsLarge.  A pure function of (T, K, E) so that the
// workspace size, the tile list and the GEMM instantiation always agree.
constexpr int kTileRowsLarge = 96;
inline int tile_rows(int T, int K, int E) { return (long)T * K <= 16L * E ? 16 : kTileRowsLarge; }

struct GroupBuffers {
    int nb;                 // grouping blocks = ceil(T / 64)
    int32_t* counts_blk;    // [nb, E]
    uint64_t* masks_blk;    // [nb, E]
    int32_t* blkoff;        // [nb, E]
    int32_t* err_blk;       // [nb]
    int32_t* scalars;       // [0] n_unique (or -1), [1] n_tiles
    int4* tiles;            // [max_tiles] (expert, row0, rows, 0)
    int max_tiles;
    int mt;                 // tile height, tile_rows(T, K, E)
    // outputs (caller's buffers for k3moe_group, workspace for forward_chunk)
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E + 1]
    int32_t* perm;          // [T * K]
    int32_t* uniq;          // [E]
};

struct ChunkWorkspace {
    GroupBuffers g;
    uint16_t* h_bf16;       // [T*K, F]  (grouped pair order)
    float* ytk;             // [T*K, D]  (pair order t*K + k)
    uint16_t* x_hi;         // [T, D]    fp32 x: bf16(x)
    uint8_t* x_lo;          // [T, ceil(D/128) * 64]  x - bf16(x) as FP4 codes, rows padded to whole steps
    uint8_t* x_los;         // [T, ceil(D/128) * 4]   their E8M0 scales
    uint16_t* x16;          // [T, D]    fp32 x: x rounded to fp16 (the fp16 items' activations)
};

int group_max_tiles(int T, int K, int E);
size_t group_workspace_bytes(int T, int K, int E, bool with_outputs);
GroupBuffers group_workspace_carve(void* ws, int T, int K, int E, bool with_outputs);
size_t chunk_workspace_bytes(int T, int K, int E, int D, int F);
ChunkWorkspace chunk_workspace_carve(void* ws, int T, int K, int E, int D, int F);

hipError_t launch_group(const int32_t* idx, int T, int K, int E, const GroupBuffers& g,
                        int32_t* n_unique_out, hipStream_t stream);
// x32 (fp32 [T, D]) or xb16 (bf16 [T, D]): exactly one is non-null.
hipError_t launch_chunk(const DevWeights& W, const float* x32, const uint16_t* xb16, int T, const int32_t* idx,
                        const float* w, int K, float* y, int32_t* n_unique_out, const ChunkWorkspace& ws,
                        hipStream_t stream);

hipError_t launch_combine(const float* ytk, const int32_t* idx, int T, int K, int D, const int32_t* scalars,
                          float* y, hipStream_t stream);

// ------------------------------------------------------------------ chunk, MXFP8 activations
struct ChunkMxWorkspace {
    GroupBuffers g;
    uint8_t* xq;            // [2][T, D]     activation codes per part
    uint8_t* xs;            // [2][T, D/32]  their scales
    uint8_t* hq;            // [2][T*K, F]   SiTU-GLU output codes (grouped pair order)
    uint8_t* hs;            // [2][T*K, F/32]
    float* ytk;             // [T*K, D]      (pair order t*K + k)
};
size_t chunk_mx_workspace_bytes(int T, int K, int E, int D, int F);
ChunkMxWorkspace chunk_mx_workspace_carve(void* ws, int T, int K, int E, int D, int F);
hipError_t launch_mx_quant(const void* v, bool bf16, size_t n, int parts, uint8_t* codes, uint8_t* scales,
                           size_t code_plane, size_t scale_plane, hipStream_t stream);
hipError_t launch_chunk_mx(const DevWeights& W, const float* x, int T, const int32_t* idx, const float* w,
                           int K, int parts, float* y, int32_t* n_unique_out, const ChunkMxWorkspace& ws,
                           hipStream_t stream);

// ------------------------------------------------------------------ dense bf16 products (LatentMoE, T >= 2)
enum { DENSE_F32 = 0, DENSE_SITU = 1 };
constexpr int kDenseMaxSplits = 16;
constexpr int kDenseMaxSplitItems = 1024;  // work items of a launch whose reduction is split
// out[T, N] = A[0] W[0]^T (+ A[1] W[1]^T over a second segment when K[1] > 0), fp32
// (DENSE_F32); or bf16 SiTU(A[0] W[0]^T, A[0] Wu^T) (DENSE_SITU, one segment).  A [T, K],
// W [N, K] row-major bf16; N and each K multiples of 32.
struct DenseProblem {
    int epi;
    const uint16_t* A[2];
    const uint16_t* W[2];
    const uint16_t* Wu;
    int K[2];
    int T, N;
    float* outf;
    uint16_t* outb;
};
struct DensePlan {
    int ms, mtiles, ntiles, splits;
};
DensePlan dense_plan(const DenseProblem& p, int slots);
size_t dense_part_bytes(int T);  // split partials of one launch
size_t dense_cnt_bytes();        // counters of one launch
// counters of ncnt launches (back to back, dense_cnt_bytes() apart) set to zero
hipError_t launch_dense_clear(int32_t* cnt, int ncnt_launches, hipStream_t stream);
hipError_t launch_dense(const DenseProblem& p, float* part, int32_t* cnt, hipStream_t stream);

// ------------------------------------------------------------------ LatentMoE block
struct LatentDims {
    int Dh, Dl, F, Fs;  // hidden width, latent width (= expert D), expert width, shared width
};
struct DevLatent {
    int Dh, Fs;
    float eps;
    const uint16_t *w_down, *w_up, *norm, *shared_gate, *shared_up, *shared_down;  // bf16
};
size_t latent_workspace_bytes(const LatentDims& L, int T, int K, int E);
hipError_t launch_latent(const DevLatent& L, const DevWeights& W, const uint16_t* h, int T, const int32_t* idx,
                         const float* w, int K, float* out, void* ws, hipStream_t stream);

// ------------------------------------------------------------------ dequant
hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int O, int I, void* out, int out_bf16,
                          hipStream_t stream);

}  // namespace k3moe
