"""Expert residency on the GPU: decode through an LRU pool of HBM slots filled from
pinned host memory matches the oracle (rel-L2 <= 1e-5, the decode tolerance) and
equals decode on fully resident weights, bit for bit; the pool's hit/miss counts
equal the placement rule's."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, torch_cuda

pytestmark = pytest.mark.gpu


def _host_slots(cfgs, used, layout, torch):
    """Pinned host [L, E, slot_bytes] in the slot layout; only the experts in
    ``used[layer]`` are filled (the pool reads no others)."""
    L, E = len(cfgs), cfgs[0].E
    host = torch.empty((L, E, layout[6]), dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()
    for li, cfg in enumerate(cfgs):
        ids = sorted(used[li])
        W = synth.weights_host(cfg, ids)
        for ti, name in enumerate(synth.TENSORS):
            a = W[name].reshape(len(ids), -1)
            hv[li, ids, layout[ti]:layout[ti] + a.shape[1]] = a
    return host


@pytest.mark.parametrize("E,K,D,F,n_slots,L", [(40, 4, 512, 256, 8, 3), (896, 16, 3584, 3072, 24, 1)])
def test_pooled_decode_equals_resident(E, K, D, F, n_slots, L):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    base = synth.CONFIGS["decode1"]
    if (E, K, D, F) == (base.E, base.K, base.D, base.F):
        cfgs = [base]
    else:
        cfgs = [synth.scaled(base, name=f"pool{E}_{li}", E=E, K=K, D=D, F=F, weight_seed=base.weight_seed + 17 * li)
                for li in range(L)]
    layout = lib.slot_layout(D, F)
    log(f"pool test: E={E} K={K} D={D} F={F} slots={n_slots} layers={L}, slot {layout[6]} B")
    # the token sequence: random layers, every fourth token repeating the previous routing
    rng = np.random.default_rng(E + K)
    toks, used = [], [set() for _ in range(L)]
    for t in range(12 if E > 100 else 30):
        li = int(rng.integers(L))
        x, logits, bias = synth.activations(cfgs[li], T=1, stream=1000 + t)
        if t % 4 == 3:
            li, logits, bias = toks[-1][0], toks[-1][4], toks[-1][5]
        idx, w, _ = oracle.route(logits, bias, K)
        used[li].update(int(e) for e in idx[0])
        toks.append((li, x[0], idx[0], w[0], logits, bias))
    host = _host_slots(cfgs, used, layout, torch)
    slots = torch.empty(n_slots * layout[6], dtype=torch.uint8, device="cuda")
    pool = lib.Pool(n_slots, D, F, slots)
    twin = lib.load().k3moe_pool_create(n_slots, D, F, ctypes.c_void_p(1 << 30))  # placement replayed on the host
    copy_stream = torch.cuda.Stream()
    resident = [device_weights(c) for c in cfgs]
    hits = misses = 0
    for t, (li, x, idx, w, _, _) in enumerate(toks):
        xd, idd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
        y_pool = lib.forward_decode_pooled(pool, li, host, host.stride(0), host.stride(1), xd, idd, wd,
                                           copy_stream=copy_stream)
        y_ref = lib.forward_decode(resident[li], xd, idd, wd)
        torch.cuda.synchronize()
        got = y_pool.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), y_ref.cpu().numpy().view(np.uint32)), t
        if E < 100 or t % 4 == 0:  # the oracle on every small-shape token and every fourth K3 token
            want = oracle_forward_subset(cfgs[li], x[None], idx[None], w[None])[0]
            assert_close(got, want, 1e-5, f"pooled decode token {t} (layer {li})")
        e = np.ascontiguousarray(idx, np.int32)
        s, m = np.empty_like(e), np.empty_like(e)
        assert lib.load().k3moe_pool_plan(twin, li, e.ctypes.data, K, s.ctypes.data, m.ctypes.data) == 0
        hits += K - int(m.sum())
        misses += int(m.sum())
    st = pool.stats()
    log(f"pool test: {st['hits']} hits, {st['misses']} misses, {st['bytes'] / 1e6:.1f} MB copied")
    assert st["hits"] == hits and st["misses"] == misses and st["bytes"] == misses * layout[6]
    lib.load().k3moe_pool_destroy(twin)
    pool.close()
