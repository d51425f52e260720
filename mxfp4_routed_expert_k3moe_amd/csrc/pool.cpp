// pool.cpp -- expert residency: an LRU pool of HBM slots filled from host memory.
//
// colibri PR #676 ("It runs the full model") and PR #684 (engine commit): the
// routed experts of all layers do not fit in fast memory, so they stream from a
// slower tier through a per-layer LRU of whole-expert slots, one read per expert
// because the six tensors of an expert are stored back to back; the loads of a
// token's misses overlap the compute of experts already loaded (K3_PIPE).  Here
// the slow tier is pinned host memory, the fast tier HBM, the read one async
// host-to-device copy per missing expert on a copy stream, and the overlap comes
// from running the gate/up products of the resident experts while the copies of
// the missing ones are in flight.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "k3moe.h"
#include "launch.hpp"

namespace {

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

// Byte offsets of gate_q, gate_s, up_q, up_s, down_q, down_s within a slot, and
// the slot size (each tensor 256-byte aligned).
void slot_layout(int32_t D, int32_t F, int64_t off[7]) {
    const size_t q = (size_t)F * D / 2, s = (size_t)F * D / 32;
    size_t o = 0;
    const size_t sizes[6] = {q, s, q, s, q, s};
    for (int i = 0; i < 6; ++i) {
        off[i] = (int64_t)o;
        o += up256(sizes[i]);
    }
    off[6] = (int64_t)o;
}

}  // namespace

struct k3moe_pool {
    int32_t n_slots = 0, D = 0, F = 0;
    int64_t off[7] = {};
    uint8_t* slots = nullptr;                  // device, n_slots * off[6] bytes (caller's)
    std::vector<int64_t> key;                  // (layer << 32 | expert) held by each slot, -1 = empty
    std::vector<uint64_t> stamp;               // last fetch that used each slot
    std::unordered_map<int64_t, int32_t> where;
    uint64_t clock = 0;
    int64_t hits = 0, misses = 0, bytes = 0;
    // device-side state, created on first use: pinned staging for slot ids, events
    int32_t* staging = nullptr;                // pinned host [3 * K3MOE_MAX_K]
    hipEvent_t copies_done = nullptr, last_done = nullptr;
    bool last_done_recorded = false;
};

namespace {

int pool_plan(k3moe_pool* P, int32_t layer, const int32_t* experts, int32_t K, int32_t* slots,
              int32_t* missed) {
    if (K > P->n_slots) return K3MOE_E_DIM;
    const uint64_t now = ++P->clock;
    // hits first, so this token's misses never evict them
    for (int32_t k = 0; k < K; ++k) {
        missed[k] = 0;
        slots[k] = K3MOE_PRUNED;
        if (experts[k] == K3MOE_PRUNED) continue;
        if (experts[k] < 0) return K3MOE_E_DIM;
        const int64_t kk = ((int64_t)layer << 32) | (uint32_t)experts[k];
        auto it = P->where.find(kk);
        if (it != P->where.end()) {
            slots[k] = it->second;
            P->stamp[it->second] = now;
        }
    }
    for (int32_t k = 0; k < K; ++k) {
        if (experts[k] == K3MOE_PRUNED || slots[k] != K3MOE_PRUNED) continue;
        const int64_t kk = ((int64_t)layer << 32) | (uint32_t)experts[k];
        auto it = P->where.find(kk);
        if (it != P->where.end()) {  // listed twice in one token: already placed
            slots[k] = it->second;
            continue;
        }
        // least recently used slot not used by this token (empty slots have stamp 0)
        int32_t victim = -1;
        for (int32_t s = 0; s < P->n_slots; ++s)
            if (P->stamp[s] != now && (victim < 0 || P->stamp[s] < P->stamp[victim])) victim = s;
        if (victim < 0) return K3MOE_E_DIM;  // cannot happen when K <= n_slots
        if (P->key[victim] >= 0) P->where.erase(P->key[victim]);
        P->key[victim] = kk;
        P->where[kk] = victim;
        P->stamp[victim] = now;
        slots[k] = victim;
        missed[k] = 1;
    }
    for (int32_t k = 0; k < K; ++k) {
        if (experts[k] == K3MOE_PRUNED) continue;
        if (missed[k]) ++P->misses;
        else ++P->hits;
    }
    return K3MOE_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? K3MOE_OK : K3MOE_E_HIP; }

}  // namespace

extern "C" {

int k3moe_slot_layout(int32_t d_model, int32_t d_ff, int64_t* offsets) {
    if (!offsets) return K3MOE_E_NULL;
    if (d_model < 32 || d_ff < 32 || d_model % 32 || d_ff % 32 || d_model > K3MOE_MAX_DIM || d_ff > K3MOE_MAX_DIM)
        return K3MOE_E_DIM;
    slot_layout(d_model, d_ff, offsets);
    return K3MOE_OK;
}

k3moe_pool_t* k3moe_pool_create(int32_t n_slots, int32_t d_model, int32_t d_ff, void* slots) {
    if (!slots || n_slots < 1 || d_model < 32 || d_ff < 32 || d_model % 32 || d_ff % 32 ||
        d_model > K3MOE_MAX_DIM || d_ff > K3MOE_MAX_DIM || (reinterpret_cast<uintptr_t>(slots) & 255))
        return nullptr;
    k3moe_pool* P = new (std::nothrow) k3moe_pool;
    if (!P) return nullptr;
    P->n_slots = n_slots;
    P->D = d_model;
    P->F = d_ff;
    slot_layout(d_model, d_ff, P->off);
    P->slots = static_cast<uint8_t*>(slots);
    P->key.assign((size_t)n_slots, -1);
    P->stamp.assign((size_t)n_slots, 0);
    return P;
}

void k3moe_pool_destroy(k3moe_pool_t* pool) {
    if (!pool) return;
    if (pool->copies_done) (void)hipEventDestroy(pool->copies_done);
    if (pool->last_done) (void)hipEventDestroy(pool->last_done);
    if (pool->staging) (void)hipHostFree(pool->staging);
    delete pool;
}

int k3moe_pool_plan(k3moe_pool_t* pool, int32_t layer, const int32_t* experts, int32_t K, int32_t* slots,
                    int32_t* missed) {
    if (!pool || !experts || !slots || !missed) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || layer < 0) return K3MOE_E_DIM;
    return pool_plan(pool, layer, experts, K, slots, missed);
}

int k3moe_pool_weights(const k3moe_pool_t* pool, k3moe_weights_t* W) {
    if (!pool || !W) return K3MOE_E_NULL;
    W->n_experts = pool->n_slots;
    W->d_model = pool->D;
    W->d_ff = pool->F;
    const uint8_t* b = pool->slots;
    W->gate_q = b + pool->off[0];
    W->gate_s = b + pool->off[1];
    W->up_q = b + pool->off[2];
    W->up_s = b + pool->off[3];
    W->down_q = b + pool->off[4];
    W->down_s = b + pool->off[5];
    W->gate_q_stride = W->gate_s_stride = W->up_q_stride = W->up_s_stride = W->down_q_stride = W->down_s_stride =
        pool->off[6];
    return K3MOE_OK;
}

int k3moe_pool_stats(const k3moe_pool_t* pool, int64_t* out) {
    if (!pool || !out) return K3MOE_E_NULL;
    out[0] = pool->hits;
    out[1] = pool->misses;
    out[2] = pool->bytes;
    return K3MOE_OK;
}

int k3moe_forward_decode_pooled(k3moe_pool_t* pool, int32_t layer, const uint8_t* host, int64_t layer_stride,
                                int64_t expert_stride, const float* x, const int32_t* idx, const float* w,
                                int32_t K, float* y, void* ws, size_t ws_bytes, void* stream_, void* copy_stream_) {
    if (!pool || !host || !x || !idx || !w || !y || !ws) return K3MOE_E_NULL;
    if (K < 1 || K > K3MOE_MAX_K || K > pool->n_slots || layer < 0 || layer_stride < 0 || expert_stride < 0)
        return K3MOE_E_DIM;
    if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(ws) & 15)) return K3MOE_E_ALIGN;
    const size_t need = k3moe::decode_workspace_bytes(K, pool->D, pool->F) + 3 * 256;
    if (ws_bytes < need) return K3MOE_E_WORKSPACE;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    hipStream_t copy_stream = static_cast<hipStream_t>(copy_stream_);
    hipError_t e;
    if (!pool->staging) {
        if ((e = hipHostMalloc(reinterpret_cast<void**>(&pool->staging), 3 * K3MOE_MAX_K * sizeof(int32_t))) !=
            hipSuccess)
            return status_of(e);
        if ((e = hipEventCreateWithFlags(&pool->copies_done, hipEventDisableTiming)) != hipSuccess) return status_of(e);
        if ((e = hipEventCreateWithFlags(&pool->last_done, hipEventDisableTiming)) != hipSuccess) return status_of(e);
    }
    // 1. the token's experts, on the host (the one synchronisation of this path)
    int32_t* experts = pool->staging;  // [K]
    if ((e = hipMemcpyAsync(experts, idx, K * sizeof(int32_t), hipMemcpyDeviceToHost, stream)) != hipSuccess)
        return status_of(e);
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return status_of(e);
    // 2. plan: slot of each expert, misses evict least recently used slots
    int32_t slots[K3MOE_MAX_K], missed[K3MOE_MAX_K];
    int rc = pool_plan(pool, layer, experts, K, slots, missed);
    if (rc != K3MOE_OK) return rc;
    // 3. copies of the misses on the copy stream, after every kernel of the previous
    //    pooled call (which may have read the evicted slots)
    if (pool->last_done_recorded && (e = hipStreamWaitEvent(copy_stream, pool->last_done, 0)) != hipSuccess)
        return status_of(e);
    int nmiss = 0;
    for (int32_t k = 0; k < K; ++k) {
        if (!missed[k]) continue;
        const uint8_t* src = host + (int64_t)layer * layer_stride + (int64_t)experts[k] * expert_stride;
        if ((e = hipMemcpyAsync(pool->slots + (size_t)slots[k] * pool->off[6], src, (size_t)pool->off[6],
                                hipMemcpyHostToDevice, copy_stream)) != hipSuccess)
            return status_of(e);
        pool->bytes += pool->off[6];
        ++nmiss;
    }
    if ((e = hipEventRecord(pool->copies_done, copy_stream)) != hipSuccess) return status_of(e);
    // 4. slot ids: all slots, resident ones only, missing ones only (pruned elsewhere);
    //    both gate/up parts take the workgroup shape the whole token would take
    //    (split rows iff the token itself has a pruned slot), so the sums match
    //    k3moe_forward_decode's bit for bit
    int split = 0;
    for (int32_t k = 0; k < K; ++k) split |= experts[k] == K3MOE_PRUNED;
    int32_t* ids = pool->staging + K3MOE_MAX_K;  // [2 * K]: hits-only, misses-only
    for (int32_t k = 0; k < K; ++k) {
        ids[k] = missed[k] ? K3MOE_PRUNED : slots[k];
        ids[K + k] = missed[k] ? slots[k] : K3MOE_PRUNED;
        experts[k] = slots[k];  // reuse: all slots
    }
    char* wsp = static_cast<char*>(ws);
    const size_t dec = k3moe::decode_workspace_bytes(K, pool->D, pool->F);
    int32_t* d_all = reinterpret_cast<int32_t*>(wsp + dec);
    int32_t* d_hit = reinterpret_cast<int32_t*>(wsp + dec + 256);
    int32_t* d_miss = reinterpret_cast<int32_t*>(wsp + dec + 512);
    if ((e = hipMemcpyAsync(d_all, experts, K * sizeof(int32_t), hipMemcpyHostToDevice, stream)) != hipSuccess ||
        (e = hipMemcpyAsync(d_hit, ids, K * sizeof(int32_t), hipMemcpyHostToDevice, stream)) != hipSuccess ||
        (e = hipMemcpyAsync(d_miss, ids + K, K * sizeof(int32_t), hipMemcpyHostToDevice, stream)) != hipSuccess)
        return status_of(e);
    // 5. gate/up of the resident experts while the copies run, then of the copied
    //    ones, then down and the combine over all slots
    k3moe_weights_t Wp;
    k3moe_pool_weights(pool, &Wp);
    k3moe::DevWeights dw;
    dw.E = Wp.n_experts;
    dw.D = Wp.d_model;
    dw.F = Wp.d_ff;
    dw.gate_q = Wp.gate_q; dw.gate_s = Wp.gate_s; dw.up_q = Wp.up_q; dw.up_s = Wp.up_s;
    dw.down_q = Wp.down_q; dw.down_s = Wp.down_s;
    dw.gate_q_stride = dw.gate_s_stride = dw.up_q_stride = dw.up_s_stride = dw.down_q_stride = dw.down_s_stride =
        Wp.gate_q_stride;
    const k3moe::DecodeWorkspace dws = k3moe::decode_workspace_carve(ws, K, dw.D, dw.F);
    if (nmiss < K &&
        (e = k3moe::launch_decode_gateup(dw, x, d_hit, K, dws.h, stream, nullptr, nullptr, split)) != hipSuccess)
        return status_of(e);
    if ((e = hipStreamWaitEvent(stream, pool->copies_done, 0)) != hipSuccess) return status_of(e);
    if (nmiss > 0 &&
        (e = k3moe::launch_decode_gateup(dw, x, d_miss, K, dws.h, stream, nullptr, nullptr, split)) != hipSuccess)
        return status_of(e);
    if ((e = k3moe::launch_decode_down(dw, dws.h, d_all, w, K, dws.ypart, y, stream)) != hipSuccess)
        return status_of(e);
    if ((e = hipEventRecord(pool->last_done, stream)) != hipSuccess) return status_of(e);
    pool->last_done_recorded = true;
    return K3MOE_OK;
}

}  // extern "C"
