// Host-side driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of
// the library's host code (every source compiled host-only, no device code): the
// argument validation of every entry point, the workspace sizing, the status
// strings, and the residency pool's slot layout and LRU planning against a plain
// reference.  Nothing here reaches a kernel launch; no GPU is needed.  Exit status
// 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <utility>
#include <vector>

#include "k3moe.h"

static int g_fail = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                    \
        }                                                                \
    } while (0)

static k3moe_weights_t weights(int D = 3584, int F = 3072, int E = 896, uintptr_t base = 1 << 20) {
    k3moe_weights_t w;
    std::memset(&w, 0, sizeof w);
    w.n_experts = E;
    w.d_model = D;
    w.d_ff = F;
    const uint8_t* p = reinterpret_cast<const uint8_t*>(base);
    w.gate_q = w.gate_s = w.up_q = w.up_s = w.down_q = w.down_s = p;
    w.gate_q_stride = w.up_q_stride = w.down_q_stride = (int64_t)F * D / 2;
    w.gate_s_stride = w.up_s_stride = w.down_s_stride = (int64_t)F * D / 32;
    return w;
}

// The reference placement: whole-expert slots; hits are refreshed first, then each
// miss takes the slot whose last use is oldest (empty slots first, equal ages: the
// lowest slot), never one this token uses.
struct RefLru {
    int n;
    std::vector<std::pair<int, int>> key;  // (layer, expert) or (-1, -1)
    std::vector<long> stamp;
    long clock = 0;
    explicit RefLru(int n_) : n(n_), key(n_, {-1, -1}), stamp(n_, 0) {}
    void token(int layer, const std::vector<int>& ex, std::vector<int>& slots, std::vector<int>& missed) {
        ++clock;
        std::vector<bool> used(n, false);
        slots.assign(ex.size(), -1);
        missed.assign(ex.size(), 0);
        for (size_t k = 0; k < ex.size(); ++k) {
            if (ex[k] < 0) continue;
            for (int s = 0; s < n; ++s)
                if (key[s] == std::make_pair(layer, ex[k])) {
                    stamp[s] = clock;
                    used[s] = true;
                    slots[k] = s;
                }
        }
        for (size_t k = 0; k < ex.size(); ++k) {
            if (ex[k] < 0 || slots[k] >= 0) continue;
            int best = -1;
            for (int s = 0; s < n; ++s) {
                if (used[s]) continue;
                const bool empty = key[s].first < 0, best_empty = best >= 0 && key[best].first < 0;
                if (best < 0 || (empty && !best_empty) || (empty == best_empty && stamp[s] < stamp[best])) best = s;
            }
            key[best] = {layer, ex[k]};
            stamp[best] = clock;
            used[best] = true;
            slots[k] = best;
            missed[k] = 1;
        }
    }
};

int main() {
    void* p = reinterpret_cast<void*>(256);
    k3moe_weights_t w = weights();
    const size_t ws = 1 << 20;

    // status strings
    for (int c = -8; c <= 1; ++c) CHECK(k3moe_status_string(c) != nullptr && std::strlen(k3moe_status_string(c)) > 0);

    // workspace sizes
    CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 1, 16, &w) >= (size_t)16 * 3072 * 4);
    CHECK(k3moe_workspace_size(K3MOE_OP_CHUNK, 4096, 16, &w) >= (size_t)4096 * 16 * 3584 * 4);
    CHECK(k3moe_workspace_size(K3MOE_OP_CHUNK_MX, 4096, 16, &w) > 0);
    CHECK(k3moe_workspace_size(K3MOE_OP_GROUP, 4096, 16, &w) > 0);
    CHECK(k3moe_workspace_size(99, 1, 16, &w) == 0);
    CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 1, 65, &w) == 0);
    CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 0, 16, &w) == 0);
    CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 1, 16, nullptr) == 0);
    k3moe_weights_t bad_d = weights(3583);
    CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 1, 16, &bad_d) == 0);
    for (int T : {1, 7, 64, 65, 1000, 4096})
        for (int K : {1, 2, 16, 64})
            for (int E : {64, 896, 4096}) {
                k3moe_weights_t x = weights(3584, 3072, E);
                CHECK(k3moe_workspace_size(K3MOE_OP_CHUNK, T, K, &x) > k3moe_workspace_size(K3MOE_OP_GROUP, T, K, &x));
            }

    // validation of every entry point (all rejected before any device call)
    CHECK(k3moe_route(nullptr, (float*)p, 1, 896, 16, (int32_t*)p, (float*)p, nullptr) == K3MOE_E_NULL);
    CHECK(k3moe_route((float*)p, (float*)p, 0, 896, 16, (int32_t*)p, (float*)p, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_route((float*)p, (float*)p, 1, 8, 9, (int32_t*)p, (float*)p, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_route_topp((float*)p, (float*)p, 1, 896, 16, 0.0 / 0.0, (int32_t*)p, (float*)p, nullptr, nullptr) ==
          K3MOE_E_DIM);
    CHECK(k3moe_forward_decode(nullptr, (float*)p, (int32_t*)p, (float*)p, 16, (float*)p, p, ws, nullptr) == K3MOE_E_NULL);
    CHECK(k3moe_forward_decode(&w, (float*)p, (int32_t*)p, (float*)p, 0, (float*)p, p, ws, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_forward_decode(&w, (float*)p, (int32_t*)p, (float*)p, 16, (float*)p, p, 100, nullptr) ==
          K3MOE_E_WORKSPACE);
    CHECK(k3moe_forward_decode(&w, (float*)260, (int32_t*)p, (float*)p, 16, (float*)p, p, ws, nullptr) == K3MOE_E_ALIGN);
    CHECK(k3moe_forward_decode(&bad_d, (float*)p, (int32_t*)p, (float*)p, 16, (float*)p, p, ws, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_forward_decode_noalloc(nullptr, (float*)p, (int32_t*)p, (float*)p, 16, (float*)p, nullptr) ==
          K3MOE_E_NULL);
    CHECK(k3moe_forward_decode_noalloc(&w, (float*)p, (int32_t*)p, (float*)p, 0, (float*)p, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_forward_decode_noalloc(&w, (float*)260, (int32_t*)p, (float*)p, 16, (float*)p, nullptr) ==
          K3MOE_E_ALIGN);
    {
        k3moe_weights_t big = weights(8192, 8192, 896);
        CHECK(k3moe_workspace_size(K3MOE_OP_DECODE, 1, 32, &big) <= K3MOE_NOALLOC_SCRATCH_BYTES);
        CHECK(k3moe_forward_decode_noalloc(&big, (float*)p, (int32_t*)p, (float*)p, 33, (float*)p, nullptr) ==
              K3MOE_E_SCRATCH);
        CHECK(std::strlen(k3moe_status_string(K3MOE_E_SCRATCH)) > 20);
    }
    CHECK(k3moe_forward_decode_timed(&w, (float*)p, (int32_t*)p, (float*)p, 16, (float*)p, p, ws, nullptr, p,
                                     nullptr) == K3MOE_E_NULL);
    CHECK(k3moe_decode_gateup(&w, nullptr, (int32_t*)p, 16, (float*)p, nullptr) == K3MOE_E_NULL);
    CHECK(k3moe_decode_down(&w, (float*)p, (int32_t*)p, (float*)p, 65, (float*)p, p, ws, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_forward_chunk(&w, (float*)p, 0, (int32_t*)p, (float*)p, 16, (float*)p, nullptr, p, ws, nullptr) ==
          K3MOE_E_DIM);
    CHECK(k3moe_forward_chunk(&w, (float*)p, 32, (int32_t*)p, (float*)p, 16, (float*)p, nullptr, p, 100, nullptr) ==
          K3MOE_E_WORKSPACE);
    CHECK(k3moe_forward_chunk(&w, nullptr, 32, (int32_t*)p, (float*)p, 16, (float*)p, nullptr, p, ws, nullptr) ==
          K3MOE_E_NULL);
    CHECK(k3moe_forward_chunk_bf16(&w, (uint16_t*)264, 32, (int32_t*)p, (float*)p, 16, (float*)p, nullptr, p, ws,
                                   nullptr) == K3MOE_E_ALIGN);
    CHECK(k3moe_forward_chunk_mx(&w, (float*)p, 32, (int32_t*)p, (float*)p, 16, 3, (float*)p, nullptr, p, ws,
                                 nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_group((int32_t*)p, 32, 16, 896, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, p, 10,
                      nullptr) == K3MOE_E_WORKSPACE);
    CHECK(k3moe_dequant_mxfp4((uint8_t*)p, (uint8_t*)p, 4, 48, p, 0, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_mx_quant(p, 0, 48, 1, (uint8_t*)p, (uint8_t*)p, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_probe_stream_read(p, 100, 8, 0, 16, (uint32_t*)p, nullptr) == K3MOE_E_DIM);
    CHECK(k3moe_probe_mfma(9, 10, 10, (float*)p, nullptr) == K3MOE_E_DIM);
    k3moe_latent_t L;
    std::memset(&L, 0, sizeof L);
    L.d_hidden = 7168;
    L.d_shared = 6144;
    L.eps = 1e-6f;
    CHECK(k3moe_latent_workspace_size(&L, 32, 16, &w) > 0);
    CHECK(k3moe_latent_forward(&L, &w, (uint16_t*)p, 1, (int32_t*)p, (float*)p, 16, (float*)p, p, ws, nullptr) ==
          K3MOE_E_NULL);  // dense weight pointers are NULL

    // pool: slot layout and LRU planning against the reference
    int64_t off[7];
    CHECK(k3moe_slot_layout(3584, 3072, off) == K3MOE_OK);
    for (int i = 0; i < 6; ++i) CHECK(off[i] % 256 == 0 && off[i + 1] > off[i]);
    CHECK(k3moe_slot_layout(100, 3072, off) != K3MOE_OK);
    CHECK(k3moe_pool_create(0, 256, 128, reinterpret_cast<void*>(1 << 30)) == nullptr);
    unsigned rng = 12345;
    auto next = [&rng]() { rng = rng * 1103515245u + 12345u; return (rng >> 8) & 0xFFFFFF; };
    for (int n_slots : {4, 16, 64}) {
        k3moe_pool_t* pool = k3moe_pool_create(n_slots, 256, 128, reinterpret_cast<void*>(1 << 30));
        CHECK(pool != nullptr);
        if (!pool) continue;
        RefLru ref(n_slots);
        long hits = 0, misses = 0;
        for (int t = 0; t < 300; ++t) {
            const int K = 1 + (int)(next() % (unsigned)std::min(n_slots, 8));
            const int layer = (int)(next() % 3);
            std::vector<int> ex;
            while ((int)ex.size() < K) {
                const int e = (int)(next() % 24);
                bool dup = false;
                for (int v : ex) dup |= v == e;
                if (!dup) ex.push_back(e);
            }
            if (t % 7 == 3) ex[0] = K3MOE_PRUNED;
            std::vector<int32_t> slots(K), missed(K);
            CHECK(k3moe_pool_plan(pool, layer, ex.data(), K, slots.data(), missed.data()) == K3MOE_OK);
            std::vector<int> rs, rm;
            ref.token(layer, ex, rs, rm);
            for (int k = 0; k < K; ++k) {
                if (ex[k] < 0) continue;
                CHECK(slots[k] == rs[k] && missed[k] == rm[k]);
                hits += !rm[k];
                misses += rm[k];
            }
        }
        int64_t st[3];
        CHECK(k3moe_pool_stats(pool, st) == K3MOE_OK);
        CHECK(st[0] == hits && st[1] == misses);
        k3moe_weights_t pw;
        CHECK(k3moe_pool_weights(pool, &pw) == K3MOE_OK && pw.n_experts == n_slots);
        std::vector<int32_t> big(n_slots + 1, 0), s2(n_slots + 1), m2(n_slots + 1);
        for (int k = 0; k <= n_slots; ++k) big[k] = k;
        CHECK(k3moe_pool_plan(pool, 0, big.data(), n_slots + 1, s2.data(), m2.data()) != K3MOE_OK);
        k3moe_pool_destroy(pool);
    }
    if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
    else std::printf("host driver: all checks passed\n");
    return g_fail ? 1 : 0;
}
