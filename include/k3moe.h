/*
 * k3moe.h -- C ABI of the MI355X (gfx950) routed-expert library for the Kimi K3
 * "Stable LatentMoE" block.
 *
 * The block (colibri PR #684, "Kimi K3: integrate coli chat, API, and Web",
 * engine commit, Stable LatentMoE bullet; colibri PR #676, "Kimi K3 engine:
 * native-MXFP4 expert streaming ...", summary bullets):
 *   1. route:   sigmoid router with a score-correction bias, top-K of E experts,
 *               weights renormalized over the raw sigmoid scores;
 *   2. per selected expert e: g = W_gate[e] x, u = W_up[e] x   (MXFP4 weights)
 *   3. h = 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25)              (SiTU-GLU)
 *   4. y_e = W_down[e] h                                       (MXFP4 weights)
 *   5. y = sum_k w_k y_{e_k}                                   (gate-weighted combine)
 *
 * MXFP4 tensors follow the compressed-tensors "mxfp4-pack-quantized" layout
 * (colibri PR #684, MXFP4-kernel commit): a matrix [O, I] is stored as packed
 * bytes [O, I/2] -- the LOW nibble holds the even column, the high nibble the odd
 * column, bit3 of a nibble is its sign, bits 2..0 an e2m1 magnitude
 * {0, .5, 1, 1.5, 2, 3, 4, 6} -- plus ue8m0 scale bytes [O, I/32], one per 32
 * consecutive inputs of a row; a weight is w = v * 2^(s-127), rounded once to
 * fp32 (subnormals kept; values >= 2^128 are +-inf; s = 255 follows the same
 * closed form, it is not NaN).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no state except a per-device property cache.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream).  No call synchronizes; results are ready when the stream is.
 *   - Return value: K3MOE_OK (0) or a negative K3MOE_E_* code.  Arguments are
 *     validated on the host BEFORE anything is launched, so on an error nothing
 *     was enqueued.  Errors inside kernels (bad device data) cannot be returned
 *     synchronously; where they are detected the documented output says so.
 *   - Calls on different streams need separate workspaces; calls that share a
 *     workspace must be ordered on one stream.
 *   - Only gfx950 devices are supported (K3MOE_E_DEVICE otherwise).
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status codes */
#define K3MOE_OK 0
#define K3MOE_E_NULL (-1)       /* a required pointer is NULL                         */
#define K3MOE_E_DIM (-2)        /* a size is out of range (see each entry point)      */
#define K3MOE_E_ALIGN (-3)      /* a pointer or expert stride is not 16-byte aligned  */
#define K3MOE_E_WORKSPACE (-4)  /* workspace smaller than k3moe_workspace_size()      */
#define K3MOE_E_DEVICE (-5)     /* current device is not gfx950                       */
#define K3MOE_E_HIP (-6)        /* the HIP runtime reported an error at launch        */
#define K3MOE_E_SCRATCH (-7)    /* the call needs more than the fixed scratch array   */

/* Limits shared by the entry points. */
#define K3MOE_MAX_K 64          /* experts per token                                  */
#define K3MOE_PRUNED (-1)       /* routing slot dropped by top-p (k3moe_route_topp)   */
#define K3MOE_MAX_E 4096        /* experts per layer                                  */
#define K3MOE_MAX_DIM 8192      /* latent width D and expert width F                  */
#define K3MOE_MAX_ROW_ELEMS (1ll << 31) /* chunk paths: T*K*max(D, F) (and for the LatentMoE
                                           block T*max(d_hidden, d_shared)) at most this many
                                           elements: the GEMM kernels address their
                                           activation rows with 32-bit byte offsets      */
#define K3MOE_NOALLOC_SCRATCH_BYTES ((2u << 20) + (64u << 10)) /* per device, k3moe_forward_decode_noalloc */

/* Workspace kinds for k3moe_workspace_size(). */
#define K3MOE_OP_DECODE 1
#define K3MOE_OP_CHUNK 2
#define K3MOE_OP_GROUP 3
#define K3MOE_OP_CHUNK_MX 4

/* Output element types for k3moe_dequant_mxfp4(). */
#define K3MOE_OUT_F32 0
#define K3MOE_OUT_BF16 1

/* input element types of k3moe_mx_quant */
#define K3MOE_IN_F32 0
#define K3MOE_IN_BF16 1

/*
 * The routed experts of one MoE layer.  For expert e (0 <= e < n_experts):
 *   gate, up: packed [d_ff, d_model/2] at gate_q + e*gate_q_stride (bytes),
 *             scales [d_ff, d_model/32] at gate_s + e*gate_s_stride;
 *   down:     packed [d_model, d_ff/2], scales [d_model, d_ff/32].
 * The strides let the same struct address stacked [E, ...] tensors or any other
 * placement of the six tensors (the pages store them back to back per expert).
 * Requirements: d_model and d_ff multiples of 32 in [32, K3MOE_MAX_DIM];
 * 1 <= n_experts <= K3MOE_MAX_E; all six base pointers and all six strides
 * 16-byte aligned (true for stacked [E, ...] tensors: every row length is a
 * multiple of 16 bytes).  The struct itself lives in host memory and is read
 * only during the call.
 */
typedef struct k3moe_weights {
    int32_t n_experts;
    int32_t d_model;  /* D: the latent width (3584 for K3) */
    int32_t d_ff;     /* F: the expert width               */
    const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
    int64_t gate_q_stride, gate_s_stride, up_q_stride, up_s_stride, down_q_stride, down_s_stride;
} k3moe_weights_t;

/*
 * Route T tokens (step 1 above).  For each token t and expert e:
 *   score = sigmoid(logits[t,e]) evaluated in double and rounded to fp32,
 *   key   = fp32(score + bias[e])  (a NaN key counts as -inf; -0 counts as +0);
 * the K largest keys are selected, equal keys going to the lower expert id, and
 * written in descending key order to idx[t, 0..K-1]; the weights are
 *   w[t,k] = sigmoid(l_{e_k}) / sum_j sigmoid(l_{e_j})   (double, rounded to fp32),
 * so the bias steers selection only and each row of w sums to one.
 * logits [T, E] fp32, bias [E] fp32, idx [T, K] int32, w [T, K] fp32 (device).
 * Requires T >= 1, 1 <= K <= min(E, K3MOE_MAX_K), E <= K3MOE_MAX_E.
 */
int k3moe_route(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K,
                int32_t *idx, float *w, void *stream);

/*
 * k3moe_route followed by top-p pruning (colibri PR #676, K3_TOPP paragraph; PR
 * #684 engine commit, K3_TOPP bullet): of each token's K selected experts, keep
 * those with the largest routing weights until their cumulative weight reaches
 * top_p, drop the low-weight tail and renormalize the kept raw scores.  Exactly:
 *   S   = sum of the K selected sigmoid scores in slot order (double);
 *   order the K slots by descending score (equal scores: lower slot first) and
 *   keep the shortest prefix whose running sum (double) reaches top_p * S, so
 *   the expert that crosses top_p is kept and at least one expert is;
 *   the kept experts stay in their slot order in idx[t, 0..m-1] with
 *   w = score / (sum of kept scores in slot order); slots m..K-1 hold
 *   K3MOE_PRUNED with weight 0; n_kept[t] = m (device int32, nullable).
 * top_p <= 0 or >= 1 keeps all K (the output equals k3moe_route's).  Every
 * entry point below skips K3MOE_PRUNED slots: no weights are read for them and
 * they contribute nothing.  A NaN top_p is rejected (K3MOE_E_DIM).
 */
int k3moe_route_topp(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K,
                     double top_p, int32_t *idx, float *w, int32_t *n_kept, void *stream);

/*
 * Group a chunk's (token, slot) pairs by expert with a counting sort (colibri
 * PR #676, chunked-prefill paragraph: the MoE loads each unique expert of a chunk
 * once; PR #684 chunked-prefill commit: position lists via counting sort).
 * Pair p = t*K + k is routed to idx[p]; K3MOE_PRUNED slots are not pairs.
 * Outputs (device, int32):
 *   counts[E]     pairs per expert;
 *   offsets[E+1]  exclusive prefix sum of counts (offsets[E] = pairs placed,
 *                 T*K when nothing is pruned);
 *   perm[T*K]     pair ids grouped by ascending expert, ascending p within one
 *                 (entries past offsets[E] are left unspecified);
 *   uniq[E]       the experts with counts > 0 in ascending order (entries past
 *                 n_unique are left unspecified);
 *   n_unique[1]   their number, or -1 if some idx is outside [0, E) or a token
 *                 lists one expert twice (the other outputs are then unspecified).
 * ws: device workspace of k3moe_workspace_size(K3MOE_OP_GROUP, T, K, W) bytes
 * (W supplies only n_experts here).  Requires T >= 1, 1 <= K <= min(E, 64).
 */
int k3moe_group(const int32_t *idx, int32_t T, int32_t K, int32_t E, int32_t *counts,
                int32_t *offsets, int32_t *perm, int32_t *uniq, int32_t *n_unique, void *ws,
                size_t ws_bytes, void *stream);

/*
 * One token through the routed experts (steps 2-5), fp32 end to end: weights
 * are decoded to fp32 exactly, dot products accumulate in fp32, SiTU-GLU runs in
 * fp32 and the combine sums w_k * y_k in slot order k = 0..K-1.  This is the
 * memory-bound decode path; every selected expert's bytes are read once.
 * x [D] fp32, idx [K] int32 (each in [0, E), distinct, or K3MOE_PRUNED),
 * w [K] fp32, y [D] fp32.  ws: k3moe_workspace_size(K3MOE_OP_DECODE, 1, K, W)
 * bytes.  Pruned slots are skipped; other out-of-range indices are not read and
 * their slots contribute NaN to y.
 */
int k3moe_forward_decode(const k3moe_weights_t *W, const float *x, const int32_t *idx,
                         const float *w, int32_t K, float *y, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * k3moe_forward_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the same kernels, arithmetic, results and errors, but the workspace is the
 * library's own fixed scratch array of K3MOE_NOALLOC_SCRATCH_BYTES per device
 * (a static device array, held by each device the library runs on until the
 * process ends) instead of a caller buffer.  Nothing is allocated: no hipMalloc,
 * no hipFree, no allocating library call.  The caller passes x, idx, w and y as
 * for k3moe_forward_decode.
 * K3MOE_E_SCRATCH if k3moe_workspace_size(K3MOE_OP_DECODE, 1, K, W) exceeds
 * K3MOE_NOALLOC_SCRATCH_BYTES (2 MiB + 64 KiB: h, the per-slot partials and the
 * combine counters of up to K = 32 at D = F = 8192, or K = 64 at the K3 shape
 * D = 3584, F = 3072), checked on the host before anything is launched.
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, no allocation); make that first call outside stream
 * capture.  Nothing in the scratch has to be zero before a call: the counters
 * the down kernel uses are cleared by the same call's gate/up kernel (a kernel
 * store, not a memset), the rest is written before it is read.  Every call
 * on one device shares that device's array: calls that overlap on one device
 * (different streams, or different host threads without ordering) race and
 * their outputs are undefined; calls ordered on one stream are safe.
 */
int k3moe_forward_decode_noalloc(const k3moe_weights_t *W, const float *x, const int32_t *idx,
                                 const float *w, int32_t K, float *y, void *stream);

/*
 * k3moe_forward_decode with its first kernel's duration recorded: ev_start and
 * ev_stop are hipEvent_t handles the caller created (hipEventCreate) and owns;
 * the gate/up + SiTU-GLU kernel (the larger of the two, 2/3 of the expert
 * bytes) is launched through hipExtLaunchKernelGGL, which records ev_start when
 * it begins and ev_stop when it ends, so hipEventElapsedTime on the pair is that
 * kernel alone (no launch or queue gap, unlike events recorded on the stream
 * around the call).  Same arguments, arithmetic and errors as
 * k3moe_forward_decode; a null event is K3MOE_E_NULL.
 */
int k3moe_forward_decode_timed(const k3moe_weights_t *W, const float *x, const int32_t *idx,
                               const float *w, int32_t K, float *y, void *ws, size_t ws_bytes,
                               void *ev_start, void *ev_stop, void *stream);

/*
 * The two stages of k3moe_forward_decode, callable apart (to read the SiTU-GLU
 * activations, or to time the stages).  Same arithmetic as forward_decode.
 * k3moe_decode_gateup (steps 2-3): h[k, f] = SiTU-GLU((W_gate[e_k] x)_f,
 *   (W_up[e_k] x)_f) for k < K, f < F; x [D] fp32, idx [K], h [K, F] fp32.
 *   An out-of-range idx[k] gives a NaN row h[k]; a pruned slot's row is not
 *   written.
 * k3moe_decode_down (steps 4-5): y[d] = sum_k w_k * (W_down[e_k] h[k])_d summed in
 *   slot order; h [K, F] fp32 (16-byte aligned), y [D] fp32; ws as for
 *   k3moe_forward_decode (it holds the per-slot down outputs).
 */
int k3moe_decode_gateup(const k3moe_weights_t *W, const float *x, const int32_t *idx, int32_t K,
                        float *h, void *stream);
int k3moe_decode_down(const k3moe_weights_t *W, const float *h, const int32_t *idx, const float *w,
                      int32_t K, float *y, void *ws, size_t ws_bytes, void *stream);

/*
 * A chunk of T tokens through the routed experts (steps 2-5) with the chunk's
 * expert union deduplicated (colibri PR #676, chunked-prefill paragraph: each
 * unique expert of a chunk is loaded once and run for every position routed to
 * it): the pairs are grouped by expert (k3moe_group), each routed expert's
 * weights are streamed once per group of up to 96 of its tokens, and gate/up and
 * down run as MFMA matrix products with fp32 accumulation.  x [T, D] is fp32.  A
 * work item (a tile of one expert's pairs and a block of output columns) whose
 * weights all decode to fp16 normals (scale bytes 114..140) multiplies on the fp16
 * MFMA: x rounded to fp16 (RNE) and h rounded to fp16 between the two products,
 * the weights exact.  Any other item (other scale bytes, or some |x| beyond the
 * fp16 range) multiplies on the bf16 MFMA: x split exactly into hi = bf16(x) and
 * lo = x - hi, hi in the bf16 product, lo (below 2^-9 |x|) in a second product in
 * MXFP4 (e2m1 codes, one power-of-two scale per 32 columns) against the weights'
 * own FP4 codes, summed into the same fp32 accumulators; its down product takes h
 * rounded to bf16.  The combine sums w_{t,k} * y_{t,k} in slot order in fp32.  The
 * result is within about 1e-3 (relative L2) of the exact block at the K3 shape
 * (1.5e-3 on the bf16 items).
 * x [T, D] fp32 (16-byte aligned), idx [T, K] int32 (K3MOE_PRUNED slots skipped),
 * w [T, K] fp32, y [T, D] fp32; n_unique (device int32, nullable) receives the
 * union size, or -1 for invalid routing, in which case every element of y is NaN.
 * ws: k3moe_workspace_size(K3MOE_OP_CHUNK, T, K, W) bytes.  T*K <= 2^30 and
 * T*K*max(D, F) <= K3MOE_MAX_ROW_ELEMS, else K3MOE_E_DIM.
 */
int k3moe_forward_chunk(const k3moe_weights_t *W, const float *x, int32_t T, const int32_t *idx,
                        const float *w, int32_t K, float *y, int32_t *n_unique, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * k3moe_forward_chunk for activations that are already bf16 (raw 16-bit
 * patterns, [T, D], 16-byte aligned): every item on the bf16 MFMA without a low
 * part, h rounded to bf16.  Same
 * arguments, workspace (K3MOE_OP_CHUNK), outputs and errors.
 */
int k3moe_forward_chunk_bf16(const k3moe_weights_t *W, const uint16_t *x, int32_t T, const int32_t *idx,
                             const float *w, int32_t K, float *y, int32_t *n_unique, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * The chunk path with MXFP8 activations (the GPU form of the pages' per-32
 * low-precision activations, colibri PR #684 int8-activation commit): x and h are
 * quantized in groups of 32 consecutive values to OCP MXFP8 (E4M3 codes, one
 * E8M0 scale byte per group; see k3moe_mx_quant) in `parts` parts (1, or 2 where
 * the second part quantizes the first's fp32 residual), and the products run on
 * the scaled FP8 x FP4 MFMA with the MXFP4 weights as stored, fp32 accumulation.
 * The weights keep the closed form for every scale byte, 255 included (2^128;
 * colibri PR #684, MXFP4-kernel commit).  x [T, D] fp32; arguments, outputs and
 * the combine as in k3moe_forward_chunk, plus parts.  Requires d_model and d_ff
 * multiples of 128.
 * ws: k3moe_workspace_size(K3MOE_OP_CHUNK_MX, T, K, W) bytes (for either parts).
 */
int k3moe_forward_chunk_mx(const k3moe_weights_t *W, const float *x, int32_t T, const int32_t *idx,
                           const float *w, int32_t K, int32_t parts, float *y, int32_t *n_unique, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * The LatentMoE block around the routed experts (colibri PR #684 engine commit,
 * Stable LatentMoE bullet: latent 7168 <-> 3584 projections around the experts,
 * RMSNorm on the aggregate, two fused shared experts, SiTU-GLU; PR #676 summary:
 * the routed experts run in the latent space behind shared down/up projections,
 * plus two fused full-width shared experts).  Dense weights are bf16 (raw 16-bit
 * patterns), row-major, owned by the caller:
 *   w_down [d_latent, d_hidden], w_up [d_hidden, d_latent], norm [d_latent],
 *   shared_gate / shared_up [d_shared, d_hidden], shared_down [d_hidden, d_shared]
 * (d_shared is the width of the two shared experts fused, both halves), eps the
 * RMSNorm epsilon.  d_latent is the routed experts' d_model.
 */
typedef struct k3moe_latent {
    int32_t d_hidden, d_shared;
    float eps;
    const uint16_t *w_down, *w_up, *norm, *shared_gate, *shared_up, *shared_down;
} k3moe_latent_t;

/*
 * One LatentMoE block for T tokens with hidden states h [T, d_hidden] (bf16):
 *   x = w_down h;  a = sum_k w_k E_k(x) (routing idx/w [T, K] as for the routed
 *   entry points, e.g. from k3moe_route on the router's logits);
 *   out = w_up RMSNorm(a) + shared_down SiTU-GLU(shared_gate h, shared_up h)
 * with RMSNorm(a) = norm * a / sqrt(mean(a^2) + eps).  out [T, d_hidden] fp32.
 * x stays fp32 (the projection's fp32 accumulation) and the routed block is
 * k3moe_forward_decode's path for T = 1 and k3moe_forward_chunk's (fp32 x)
 * otherwise; RMSNorm and SiTU-GLU outputs are bf16; the dense products are bf16
 * x bf16 with fp32 accumulation (this library's GEMV kernels for T = 1, its MFMA
 * GEMM kernels otherwise, whose split reductions are summed in a fixed order: the
 * output does not depend on scheduling).
 * Requires d_hidden and d_shared multiples of 32 in [32, K3MOE_MAX_DIM], eps >= 0,
 * every pointer 16-byte aligned.  ws: k3moe_latent_workspace_size() bytes; the
 * call allocates nothing.
 */
int k3moe_latent_forward(const k3moe_latent_t *L, const k3moe_weights_t *W, const uint16_t *h, int32_t T,
                         const int32_t *idx, const float *w, int32_t K, float *out, void *ws, size_t ws_bytes,
                         void *stream);

/* Bytes of device workspace for k3moe_latent_forward; 0 for invalid arguments.
 * Pure host function. */
size_t k3moe_latent_workspace_size(const k3moe_latent_t *L, int32_t T, int32_t K, const k3moe_weights_t *W);

/*
 * OCP MXFP8 quantization as the MX chunk path does it, on n values (n a positive
 * multiple of 32) of fp32 (in_dtype K3MOE_IN_F32) or bf16 (K3MOE_IN_BF16, raw
 * 16-bit patterns).  For each group of 32 with largest magnitude amax: scale byte
 * s = max(floor(log2 amax) - 8 + 127, 0), codes = the values times 2^(127-s),
 * clamped to +-448, rounded to the nearest E4M3 value, ties to even, sign kept;
 * an all-zero group gets s = 0, a group holding a NaN or an infinity s = 255 and
 * codes 0x7F.  With parts = 2 the second part quantizes the exact fp32 residual
 * v - value(part 0) the same way.  codes [parts][n] and scales [parts][n/32]
 * (device, part planes back to back); v and codes 16-byte aligned.
 */
int k3moe_mx_quant(const void *v, int32_t in_dtype, int64_t n, int32_t parts, uint8_t *codes, uint8_t *scales,
                   void *stream);

/*
 * Expert residency (colibri PR #676, "It runs the full model"; PR #684 engine
 * commit: routed experts stream through a per-layer LRU of whole-expert slots,
 * one read per expert because its six tensors sit back to back, with the reads
 * of a token's misses overlapping the compute of experts already loaded).  Here
 * the slow tier is pinned host memory and the slots live in HBM.
 *
 * k3moe_slot_layout: byte offsets of gate_q, gate_s, up_q, up_s, down_q, down_s
 *   within one slot (offsets[0..5], each 256-byte aligned) and the slot size
 *   (offsets[6]).  Host experts must use the same layout, at host + layer *
 *   layer_stride + expert * expert_stride.  Pure host function.
 * k3moe_pool_create: a pool of n_slots slots over caller-owned device memory
 *   `slots` (n_slots * offsets[6] bytes, 256-byte aligned); returns NULL on bad
 *   arguments.  The pool is a host object; it allocates a small pinned staging
 *   buffer and two events on first use (released by k3moe_pool_destroy).  One
 *   host thread at a time may use a pool.
 * k3moe_pool_plan: the placement step alone (no device work): for a token's K
 *   experts of `layer` (host int32, K3MOE_PRUNED skipped) writes the slot of each
 *   (slots[K], host) and whether it had to be loaded (missed[K]); hits are
 *   refreshed first, each miss evicts the least recently used slot not used by
 *   this token.  Requires K <= n_slots.
 * k3moe_pool_weights: a k3moe_weights_t addressing the slots as n_slots experts.
 * k3moe_pool_stats: out[0] hits, out[1] misses, out[2] bytes copied.
 * k3moe_forward_decode_pooled: k3moe_forward_decode for one token of `layer`
 *   whose experts live in host memory: copies idx (device, [K]) to the host and
 *   waits for `stream` (the one host synchronisation), plans the slots, issues
 *   one host-to-device copy per missing expert on copy_stream (after the kernels
 *   of the previous pooled call, which may still read evicted slots), runs the
 *   gate/up products of the resident experts on `stream` while the copies run,
 *   then those of the copied experts, then down and the combine.  The output
 *   equals k3moe_forward_decode's on the same experts bit for bit.  ws:
 *   k3moe_workspace_size(K3MOE_OP_DECODE, 1, K, W) + 768 bytes.
 */
typedef struct k3moe_pool k3moe_pool_t;
int k3moe_slot_layout(int32_t d_model, int32_t d_ff, int64_t *offsets);
k3moe_pool_t *k3moe_pool_create(int32_t n_slots, int32_t d_model, int32_t d_ff, void *slots);
void k3moe_pool_destroy(k3moe_pool_t *pool);
int k3moe_pool_plan(k3moe_pool_t *pool, int32_t layer, const int32_t *experts, int32_t K, int32_t *slots,
                    int32_t *missed);
int k3moe_pool_weights(const k3moe_pool_t *pool, k3moe_weights_t *W);
int k3moe_pool_stats(const k3moe_pool_t *pool, int64_t *out);
int k3moe_forward_decode_pooled(k3moe_pool_t *pool, int32_t layer, const uint8_t *host, int64_t layer_stride,
                                int64_t expert_stride, const float *x, const int32_t *idx, const float *w,
                                int32_t K, float *y, void *ws, size_t ws_bytes, void *stream, void *copy_stream);

/*
 * Bytes of device workspace needed by `op` (K3MOE_OP_*) for T tokens and K slots
 * per token on the layer described by W (n_experts, d_model, d_ff are read).
 * Returns 0 for invalid arguments.  Pure host function.
 */
size_t k3moe_workspace_size(int32_t op, int32_t T, int32_t K, const k3moe_weights_t *W);

/*
 * Decode one MXFP4 matrix (q [O, I/2], s [O, I/32]) to out [O, I] as fp32
 * (out_dtype K3MOE_OUT_F32) or bf16 (K3MOE_OUT_BF16), with the same device code
 * the matrix products use.  Every decoded value is exactly representable in both
 * types.  Requires O >= 1, I a positive multiple of 32, q 16-byte aligned.
 */
int k3moe_dequant_mxfp4(const uint8_t *q, const uint8_t *s, int32_t O, int32_t I, void *out,
                        int32_t out_dtype, void *stream);

/*
 * Measurement probes (not part of the block; the benchmark reports their rates as
 * the achievable peaks beside MI355X's published ones).
 * k3moe_probe_stream_read: reads `bytes` (a multiple of 16, buf 16-byte aligned)
 *   with `blocks` workgroups of 256 threads, each thread keeping `unroll` (4, 8
 *   or 16) 16-byte loads in flight, as ordinary or (nontemporal != 0)
 *   non-temporal loads; writes one dword per workgroup to sink[blocks] (device).
 * k3moe_probe_mfma: `blocks` workgroups of four waves, each issuing `iters`
 *   rounds of eight independent MFMAs of one kind (0: v_mfma_f32_16x16x32_bf16,
 *   16384 flops each; 1: v_mfma_scale_f32_16x16x128_f8f6f4 with FP8 E4M3 x FP4,
 *   2: FP4 x FP4, 3: FP8 x FP8, 65536 flops each; 4: v_mfma_f32_32x32x16_bf16,
 *   32768 flops; 5: v_mfma_scale_f32_32x32x64_f8f6f4 FP4 x FP4, 6: FP8 x FP4,
 *   131072 flops each); writes one float per wave to out[4 * blocks] (device).
 */
int k3moe_probe_stream_read(const void *buf, size_t bytes, int32_t unroll, int32_t nontemporal, int32_t blocks,
                            uint32_t *sink, void *stream);
int k3moe_probe_mfma(int32_t kind, int32_t iters, int32_t blocks, float *out, void *stream);

/* Text for a status code (static storage; for K3MOE_E_HIP it includes the HIP
 * runtime's message for the calling thread's last failure). */
const char *k3moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* K3MOE_H */
