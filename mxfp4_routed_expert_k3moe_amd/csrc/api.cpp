// api.cpp -- the C ABI declared in include/k3moe.h: argument validation (pure host
// code, before anything is launched), the gfx950 device check, workspace carving
// and the kernel launches on the caller's stream.  Nothing here allocates device
// memory or synchronizes.
#include <algorithm>

#include "k3moe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "launch.hpp"

namespace {

using k3moe::DevWeights;

thread_local char g_hip_msg[256] = "";

int hip_fail(hipError_t err) {
    std::snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error: %s", hipGetErrorString(err));
    return K3MOE_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int32_t v) { return v >= 32 && v <= K3MOE_MAX_DIM && v % 32 == 0; }

int check_weights(const k3moe_weights_t* W) {
    if (!W) return K3MOE_E_NULL;
    if (!W->gate_q || !W->gate_s || !W->up_q || !W->up_s || !W->down_q || !W->down_s) return K3MOE_E_NULL;
    if (W->n_experts < 1 || W->n_experts > K3MOE_MAX_E || !dim_ok(W->d_model) || !dim_ok(W->d_ff))
        return K3MOE_E_DIM;
    if (!aligned16(W->gate_q) || !aligned16(W->up_q) || !aligned16(W->down_q) || !aligned16(W->gate_s) ||
        !aligned16(W->up_s) || !aligned16(W->down_s))
        return K3MOE_E_ALIGN;
    if ((W->gate_q_stride | W->up_q_stride | W->down_q_stride | W->gate_s_stride | W->up_s_stride |
         W->down_s_stride) & 15)
        return K3MOE_E_ALIGN;
    if (W->gate_q_stride < 0 || W->up_q_stride < 0 || W->down_q_stride < 0 || W->gate_s_stride < 0 ||
        W->up_s_stride < 0 || W->down_s_stride < 0)
        return K3MOE_E_DIM;
    return K3MOE_OK;
}

DevWeights dev_weights(const k3moe_weights_t* W) {
    DevWeights d;
    d.E = W->n_experts;
    d.D = W->d_model;
    d.F = W->d_ff;
    d.gate_q = W->gate_q; d.gate_s = W->gate_s;
    d.up_q = W->up_q; d.up_s = W->up_s;
    d.down_q = W->down_q; d.down_s = W->down_s;
    d.gate_q_stride = W->gate_q_stride; d.gate_s_stride = W->gate_s_stride;
    d.up_q_stride = W->up_q_stride; d.up_s_stride = W->up_s_stride;
    d.down_q_stride = W->down_q_stride; d.down_s_stride = W->down_s_stride;
    return d;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

int check_device() {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err);
    if (dev < 0 || dev >= kMaxDevices) return K3MOE_E_DEVICE;
    int state = g_dev_ok[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        err = hipGetDeviceProperties(&prop, dev);
        if (err != hipSuccess) return hip_fail(err);
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_ok[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? K3MOE_OK : K3MOE_E_DEVICE;
}

int finish(hipError_t err) { return err == hipSuccess ? K3MOE_OK : hip_fail(err); }

}  // namespace

extern "C" {

int k3moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K, int32_t* idx,
                float* w, void* stream) {
    if (!logits || !bias || !idx || !w) return K3MOE_E_NULL;
    if (T < 1 || E < 1 || E > K3MOE_MAX_E || K < 1 || K > E || K > K3MOE_MAX_K) return K3MOE_E_DIM;
    int rc = check_device();
    if (rc != K3MOE_OK) return rc;
    return finish(k3moe::launch_route(logits, bias, T, E, K, 0.0, idx, w, nullptr, static_cast<hipStream_t>(stream)));
}

int k3moe_route_topp(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K, double top_p,
                     int32_t* idx, float* w, int32_t* n_kept, void* stream) {
    if (!logits || !bias || !idx || !w) return K3MOE_E_NULL;
    if (T < 1 || E < 1 || E > K3MOE_MAX_E || K < 1 || K > E || K > K3MOE_MAX_K) return K3MOE_E_DIM;
    if (top_p != top_p) return K3MOE_E_DIM;  // NaN
    int rc = check_device();
    if (rc != K3MOE_OK) return rc;
    return finish(k3moe::launch_route(logits, bias, T, E, K, top_p, idx, w, n_kept, static_cast<hipStream_t>(stream)));
}

size_t k3moe_workspace_size(int32_t op, int32_t T, int32_t K, const k3moe_weights_t* W) {
    if (!W || T < 1 || K < 1 || K > K3MOE_MAX_K || W->n_experts < 1 || W->n_experts > K3MOE_MAX_E ||
        K > W->n_experts)
        return 0;
    switch (op) {
        case K3MOE_OP_DECODE:
            if (!dim_ok(W->d_model) || !dim_ok(W->d_ff)) return 0;
            return k3moe::decode_workspace_bytes(K, W->d_model, W->d_ff);
        case K3MOE_OP_CHUNK:
            if (!dim_ok(W->d_model) || !dim_ok(W->d_ff)) return 0;
            return k3moe::chunk_workspace_bytes(T, K, W->n_experts, W->d_model, W->d_ff);
        case K3MOE_OP_GROUP:
            return k3moe::group_workspace_bytes(T, K, W->n_experts, false);
        case K3MOE_OP_CHUNK_MX:
            if (!dim_ok(W->d_model) || !dim_ok(W->d_ff) || W->d_model % 128 || W->d_ff % 128) return 0;
            return k3moe::chunk_mx_workspace_bytes(T, K, W->n_experts, W->d_model, W->d_ff);
        default:
            return 0;
    }
}

int k3moe_group(const int32_t* idx, int32_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* uniq, int32_t* n_unique, void* ws, size_t ws_bytes, void* stream) {
    if (!idx || !counts || !offsets || !perm || !uniq || !n_unique || !ws) return K3MOE_E_NULL;
    if (T < 1 || E < 1 || E > K3MOE_MAX_E || K < 1 || K > E || K > K3MOE_MAX_K) return K3MOE_E_DIM;
    if ((long long)T * K > (1ll << 30)) return K3MOE_E_DIM;
    if (!aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::group_workspace_bytes(T, K, E, false)) return K3MOE_E_WORKSPACE;
    int rc = check_device();
    if (rc != K3MOE_OK) return rc;
    k3moe::GroupBuffers g = k3moe::group_workspace_carve(ws, T, K, E, false);
    g.counts = counts;
    g.offsets = offsets;
    g.perm = perm;
    g.uniq = uniq;
    return finish(k3moe::launch_group(idx, T, K, E, g, n_unique, static_cast<hipStream_t>(stream)));
}

int k3moe_forward_decode(const k3moe_weights_t* W, const float* x, const int32_t* idx, const float* w,
                         int32_t K, float* y, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !w || !y || !ws) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (!aligned16(x) || !aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::decode_workspace_bytes(K, W->d_model, W->d_ff)) return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const DevWeights dw = dev_weights(W);
    const k3moe::DecodeWorkspace dws = k3moe::decode_workspace_carve(ws, K, dw.D, dw.F);
    return finish(k3moe::launch_decode(dw, x, idx, w, K, y, dws, static_cast<hipStream_t>(stream)));
}

int k3moe_forward_decode_noalloc(const k3moe_weights_t* W, const float* x, const int32_t* idx, const float* w,
                                 int32_t K, float* y, void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !w || !y) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (!aligned16(x)) return K3MOE_E_ALIGN;
    if (k3moe::decode_workspace_bytes(K, W->d_model, W->d_ff) > K3MOE_NOALLOC_SCRATCH_BYTES) return K3MOE_E_SCRATCH;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    void* ws = nullptr;
    hipError_t err = k3moe::noalloc_scratch(&ws);
    if (err != hipSuccess) return hip_fail(err);
    const DevWeights dw = dev_weights(W);
    const k3moe::DecodeWorkspace dws = k3moe::decode_workspace_carve(ws, K, dw.D, dw.F);
    return finish(k3moe::launch_decode(dw, x, idx, w, K, y, dws, static_cast<hipStream_t>(stream)));
}

int k3moe_forward_decode_timed(const k3moe_weights_t* W, const float* x, const int32_t* idx, const float* w,
                               int32_t K, float* y, void* ws, size_t ws_bytes, void* ev_start, void* ev_stop,
                               void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !w || !y || !ws || !ev_start || !ev_stop) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (!aligned16(x) || !aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::decode_workspace_bytes(K, W->d_model, W->d_ff)) return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const DevWeights dw = dev_weights(W);
    const k3moe::DecodeWorkspace dws = k3moe::decode_workspace_carve(ws, K, dw.D, dw.F);
    return finish(k3moe::launch_decode(dw, x, idx, w, K, y, dws, static_cast<hipStream_t>(stream),
                                       static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)));
}

int k3moe_decode_gateup(const k3moe_weights_t* W, const float* x, const int32_t* idx, int32_t K, float* h,
                        void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !h) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (!aligned16(x)) return K3MOE_E_ALIGN;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    return finish(k3moe::launch_decode_gateup(dev_weights(W), x, idx, K, h, static_cast<hipStream_t>(stream)));
}

int k3moe_decode_down(const k3moe_weights_t* W, const float* h, const int32_t* idx, const float* w, int32_t K,
                      float* y, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!h || !idx || !w || !y || !ws) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (!aligned16(h) || !aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::decode_workspace_bytes(K, W->d_model, W->d_ff)) return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const DevWeights dw = dev_weights(W);
    const k3moe::DecodeWorkspace dws = k3moe::decode_workspace_carve(ws, K, dw.D, dw.F);
    return finish(k3moe::launch_decode_down(dw, h, idx, w, K, dws.ypart, y, static_cast<hipStream_t>(stream)));
}

// The chunk GEMMs address activation rows (x by token, h by pair) with 32-bit
// byte offsets: T*K*max(D, F) 16-bit elements must stay within 2^32 bytes.
static bool chunk_rows_ok(int32_t T, int32_t K, const k3moe_weights_t* W) {
    return (long long)T * K * std::max(W->d_model, W->d_ff) <= K3MOE_MAX_ROW_ELEMS;
}

static int forward_chunk_any(const k3moe_weights_t* W, const float* x32, const uint16_t* xb16, int32_t T,
                             const int32_t* idx, const float* w, int32_t K, float* y, int32_t* n_unique, void* ws,
                             size_t ws_bytes, void* stream) {
    const void* x = x32 ? static_cast<const void*>(x32) : static_cast<const void*>(xb16);
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !w || !y || !ws) return K3MOE_E_NULL;
    if (T < 1 || K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if ((long long)T * K > (1ll << 30) || !chunk_rows_ok(T, K, W)) return K3MOE_E_DIM;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::chunk_workspace_bytes(T, K, W->n_experts, W->d_model, W->d_ff))
        return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const DevWeights dw = dev_weights(W);
    const k3moe::ChunkWorkspace cws = k3moe::chunk_workspace_carve(ws, T, K, dw.E, dw.D, dw.F);
    return finish(
        k3moe::launch_chunk(dw, x32, xb16, T, idx, w, K, y, n_unique, cws, static_cast<hipStream_t>(stream)));
}

int k3moe_forward_chunk(const k3moe_weights_t* W, const float* x, int32_t T, const int32_t* idx, const float* w,
                        int32_t K, float* y, int32_t* n_unique, void* ws, size_t ws_bytes, void* stream) {
    if (!x) return K3MOE_E_NULL;
    return forward_chunk_any(W, x, nullptr, T, idx, w, K, y, n_unique, ws, ws_bytes, stream);
}

int k3moe_forward_chunk_bf16(const k3moe_weights_t* W, const uint16_t* x, int32_t T, const int32_t* idx,
                             const float* w, int32_t K, float* y, int32_t* n_unique, void* ws, size_t ws_bytes,
                             void* stream) {
    if (!x) return K3MOE_E_NULL;
    return forward_chunk_any(W, nullptr, x, T, idx, w, K, y, n_unique, ws, ws_bytes, stream);
}

int k3moe_forward_chunk_mx(const k3moe_weights_t* W, const float* x, int32_t T, const int32_t* idx,
                           const float* w, int32_t K, int32_t parts, float* y, int32_t* n_unique, void* ws,
                           size_t ws_bytes, void* stream) {
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!x || !idx || !w || !y || !ws) return K3MOE_E_NULL;
    if (T < 1 || K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if (parts != 1 && parts != 2) return K3MOE_E_DIM;
    if (W->d_model % 128 || W->d_ff % 128) return K3MOE_E_DIM;
    if ((long long)T * K > (1ll << 30) || !chunk_rows_ok(T, K, W)) return K3MOE_E_DIM;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe::chunk_mx_workspace_bytes(T, K, W->n_experts, W->d_model, W->d_ff))
        return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const DevWeights dw = dev_weights(W);
    const k3moe::ChunkMxWorkspace cws = k3moe::chunk_mx_workspace_carve(ws, T, K, dw.E, dw.D, dw.F);
    return finish(k3moe::launch_chunk_mx(dw, x, T, idx, w, K, parts, y, n_unique, cws,
                                         static_cast<hipStream_t>(stream)));
}

static bool latent_ok(const k3moe_latent_t* L, const k3moe_weights_t* W) {
    return L && W && dim_ok(L->d_hidden) && dim_ok(L->d_shared) && L->eps >= 0.0f && dim_ok(W->d_model) &&
           dim_ok(W->d_ff) && W->n_experts >= 1 && W->n_experts <= K3MOE_MAX_E;
}

size_t k3moe_latent_workspace_size(const k3moe_latent_t* L, int32_t T, int32_t K, const k3moe_weights_t* W) {
    if (!latent_ok(L, W) || T < 1 || K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return 0;
    const k3moe::LatentDims d{L->d_hidden, W->d_model, W->d_ff, L->d_shared};
    return k3moe::latent_workspace_bytes(d, T, K, W->n_experts);
}

int k3moe_latent_forward(const k3moe_latent_t* L, const k3moe_weights_t* W, const uint16_t* h, int32_t T,
                         const int32_t* idx, const float* w, int32_t K, float* out, void* ws, size_t ws_bytes,
                         void* stream) {
    if (!L) return K3MOE_E_NULL;
    int rc = check_weights(W);
    if (rc != K3MOE_OK) return rc;
    if (!h || !idx || !w || !out || !ws || !L->w_down || !L->w_up || !L->norm || !L->shared_gate ||
        !L->shared_up || !L->shared_down)
        return K3MOE_E_NULL;
    if (!latent_ok(L, W) || T < 1 || K < 1 || K > K3MOE_MAX_K || K > W->n_experts) return K3MOE_E_DIM;
    if ((long long)T * K > (1ll << 30) || !chunk_rows_ok(T, K, W) ||
        (long long)T * std::max(L->d_hidden, L->d_shared) > K3MOE_MAX_ROW_ELEMS)
        return K3MOE_E_DIM;
    if (!aligned16(h) || !aligned16(out) || !aligned16(ws) || !aligned16(L->w_down) || !aligned16(L->w_up) ||
        !aligned16(L->norm) || !aligned16(L->shared_gate) || !aligned16(L->shared_up) || !aligned16(L->shared_down))
        return K3MOE_E_ALIGN;
    if (ws_bytes < k3moe_latent_workspace_size(L, T, K, W)) return K3MOE_E_WORKSPACE;
    rc = check_device();
    if (rc != K3MOE_OK) return rc;
    const k3moe::DevLatent dl{L->d_hidden, L->d_shared, L->eps, L->w_down, L->w_up, L->norm,
                              L->shared_gate, L->shared_up, L->shared_down};
    return finish(k3moe::launch_latent(dl, dev_weights(W), h, T, idx, w, K, out, ws,
                                       static_cast<hipStream_t>(stream)));
}

int k3moe_mx_quant(const void* v, int32_t in_dtype, int64_t n, int32_t parts, uint8_t* codes, uint8_t* scales,
                   void* stream) {
    if (!v || !codes || !scales) return K3MOE_E_NULL;
    if (n < 32 || n % 32 != 0 || (parts != 1 && parts != 2)) return K3MOE_E_DIM;
    if (in_dtype != K3MOE_IN_F32 && in_dtype != K3MOE_IN_BF16) return K3MOE_E_DIM;
    if (!aligned16(v) || !aligned16(codes)) return K3MOE_E_ALIGN;
    int rc = check_device();
    if (rc != K3MOE_OK) return rc;
    return finish(k3moe::launch_mx_quant(v, in_dtype == K3MOE_IN_BF16, (size_t)n, parts, codes, scales, (size_t)n,
                                         (size_t)n / 32, static_cast<hipStream_t>(stream)));
}

int k3moe_dequant_mxfp4(const uint8_t* q, const uint8_t* s, int32_t O, int32_t I, void* out,
                        int32_t out_dtype, void* stream) {
    if (!q || !s || !out) return K3MOE_E_NULL;
    if (O < 1 || I < 32 || I % 32 != 0) return K3MOE_E_DIM;
    if (out_dtype != K3MOE_OUT_F32 && out_dtype != K3MOE_OUT_BF16) return K3MOE_E_DIM;
    if (!aligned16(q) || !aligned16(out)) return K3MOE_E_ALIGN;
    int rc = check_device();
    if (rc != K3MOE_OK) return rc;
    return finish(k3moe::launch_dequant(q, s, O, I, out, out_dtype == K3MOE_OUT_BF16,
                                        static_cast<hipStream_t>(stream)));
}

const char* k3moe_status_string(int status) {
    switch (status) {
        case K3MOE_OK: return "ok";
        case K3MOE_E_NULL: return "a required pointer is NULL";
        case K3MOE_E_DIM: return "a size is out of range";
        case K3MOE_E_ALIGN: return "a pointer or expert stride is not 16-byte aligned";
        case K3MOE_E_WORKSPACE: return "workspace smaller than k3moe_workspace_size()";
        case K3MOE_E_DEVICE: return "the current device is not gfx950";
        case K3MOE_E_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
        case K3MOE_E_SCRATCH:
            return "the call needs more device scratch than K3MOE_NOALLOC_SCRATCH_BYTES (use the entry point that takes "
                   "a workspace)";
        default: return "unknown status";
    }
}

}  // extern "C"
