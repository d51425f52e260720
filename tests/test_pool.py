"""Expert residency pool on the CPU: slot layout, LRU placement against a plain
reference, statistics and argument checks (no device work)."""
import ctypes
import numpy as np

from mxfp4_routed_expert_k3moe_amd import lib as k3

FAKE_SLOTS = ctypes.c_void_p(1 << 30)  # never dereferenced by planning


def _pool(n_slots, D=256, F=128):
    L = k3.load()
    h = L.k3moe_pool_create(n_slots, D, F, FAKE_SLOTS)
    assert h
    return L, h


def _plan(L, h, layer, experts):
    e = np.ascontiguousarray(experts, dtype=np.int32)
    s = np.empty_like(e)
    m = np.empty_like(e)
    rc = L.k3moe_pool_plan(h, layer, e.ctypes.data, e.size, s.ctypes.data, m.ctypes.data)
    return rc, s, m


class RefLRU:
    """Whole-expert slots; a miss takes the slot whose last use is oldest (empty
    slots first; equal ages: lowest slot), never one this token uses."""

    def __init__(self, n):
        self.n, self.key, self.stamp, self.clock = n, [None] * n, [0] * n, 0

    def token(self, layer, experts):
        self.clock += 1
        where = {k: s for s, k in enumerate(self.key) if k is not None}
        keys = [(layer, int(e)) for e in experts]
        for k in keys:
            if k in where:
                self.stamp[where[k]] = self.clock
        slots, missed = [], []
        for k in keys:
            if k in where:
                slots.append(where[k])
                missed.append(0)
                continue
            s = min((st, i) for i, st in enumerate(self.stamp) if st != self.clock)[1]
            if self.key[s] is not None:
                del where[self.key[s]]
            self.key[s], self.stamp[s] = k, self.clock
            where[k] = s
            slots.append(s)
            missed.append(1)
        return slots, missed


def test_slot_layout():
    off = (ctypes.c_int64 * 7)()
    assert k3.load().k3moe_slot_layout(3584, 3072, off) == 0
    q, s = 3072 * 3584 // 2, 3072 * 3584 // 32
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    want = [0, up(q), up(q) + up(s), 2 * up(q) + up(s), 2 * up(q) + 2 * up(s), 3 * up(q) + 2 * up(s),
            3 * up(q) + 3 * up(s)]
    assert list(off) == want and off[6] == 17547264  # K3: six tensors already 256-aligned
    assert k3.load().k3moe_slot_layout(100, 128, off) == k3.K3MOE_E_DIM


def test_lru_matches_reference():
    rng = np.random.default_rng(3)
    for n_slots, K, E, layers in [(16, 4, 40, 1), (33, 16, 128, 3), (64, 16, 896, 2)]:
        L, h = _pool(n_slots)
        ref = RefLRU(n_slots)
        hits = misses = 0
        for step in range(300):
            layer = int(rng.integers(layers))
            experts = rng.choice(min(E, 2 * n_slots) if step % 3 else E, size=K, replace=False)
            rc, s, m = _plan(L, h, layer, experts)
            assert rc == 0
            rs, rm = ref.token(layer, experts)
            assert m.tolist() == rm and s.tolist() == rs, step
            assert len(set(s.tolist())) == K
            hits += K - int(m.sum())
            misses += int(m.sum())
        st = (ctypes.c_int64 * 3)()
        L.k3moe_pool_stats(h, st)
        assert st[0] == hits and st[1] == misses
        L.k3moe_pool_destroy(h)


def test_pruned_and_errors():
    L, h = _pool(8)
    rc, s, m = _plan(L, h, 0, [5, -1, 7, -1])
    assert rc == 0 and s[1] == -1 and s[3] == -1 and m.tolist() == [1, 0, 1, 0]
    rc, s, m = _plan(L, h, 0, [7, 5])
    assert rc == 0 and m.tolist() == [0, 0]
    assert _plan(L, h, 0, list(range(9)))[0] == k3.K3MOE_E_DIM  # more experts than slots
    assert _plan(L, h, 0, [3, -2])[0] == k3.K3MOE_E_DIM
    L.k3moe_pool_destroy(h)
    assert not L.k3moe_pool_create(0, 256, 128, FAKE_SLOTS)
    assert not L.k3moe_pool_create(4, 250, 128, FAKE_SLOTS)
    assert not L.k3moe_pool_create(4, 256, 128, ctypes.c_void_p((1 << 30) + 16))  # not 256-aligned
