"""The router's threshold pass, restated on the host: with Kw = ceil(K/4), each of
the 4 waves takes T_w = the Kw-th largest key it holds, found in rounds of a wave
maximum over the lanes' best remaining keys (each round counts every lane whose
best equals the maximum once, then retires all of those lanes' codes of that key;
0 when the wave runs out), and T = min_w T_w.  The pool of codes with key >= T
always holds the exact top K, and at least K codes.  Brute force over random,
tied, flat and adversarial key sets with the kernel's expert-to-lane layout (wave
w holds experts [w*Q, (w+1)*Q), lane l of it the ones with (e - w*Q) % 64 == l),
plus the pool sizes the 16-of-896 workloads see (the kernel ranks at most 128
codes, with one wave when there are at most 64, and falls back to K rounds of wave
maxima beyond 128)."""
import numpy as np
import pytest


def codes_of(keys):
    """Unique 64-bit-like ranking codes: larger key first, then lower id (as the kernel's
    (key bits << 32) | ~id); returned as a rank order where a larger value ranks higher."""
    E = len(keys)
    order = np.lexsort((np.arange(E), -keys))  # descending key, then ascending id
    code = np.empty(E, np.int64)
    code[order] = np.arange(E, 0, -1)  # best gets E, worst gets 1 (0 = absent)
    return code


def threshold_pool(keys, K):
    E = len(keys)
    Q = (E + 3) // 4
    Kw = (K + 3) // 4
    tws = []
    for w in range(4):
        lanes = [[keys[e] for e in range(w * Q + l, min(E, (w + 1) * Q), 64)] for l in range(64)]
        tw, counted = None, 0
        for _ in range(Kw):
            heads = [max(v) if v else None for v in lanes]
            live = [h for h in heads if h is not None]
            if not live:
                break  # fewer than Kw codes in this wave: no bound
            m = max(live)
            hit = [l for l in range(64) if heads[l] is not None and heads[l] == m]
            counted += len(hit)
            if counted >= Kw:
                tw = m
                break
            for l in hit:
                lanes[l] = [v for v in lanes[l] if v != m]
        tws.append(tw)
    if any(t is None for t in tws):
        return np.arange(E)
    T = min(tws)
    return np.nonzero(keys >= T)[0]


def check(keys, K):
    code = codes_of(keys)
    pool = threshold_pool(keys, K)
    top = np.argsort(-code, kind="stable")[:K]
    assert len(pool) >= K
    assert set(top.tolist()) <= set(pool.tolist())
    # ranking the pool by code gives the exact selection in order
    sel = pool[np.argsort(-code[pool], kind="stable")][:K]
    assert np.array_equal(sel, top)
    return len(pool)


@pytest.mark.parametrize("E,K", [(8, 2), (20, 1), (64, 64), (100, 33), (300, 1), (896, 16), (896, 1), (2000, 20),
                                 (4096, 16), (4096, 64)])
def test_pool_holds_top_k(E, K):
    rng = np.random.default_rng(E * 131 + K)
    for trial in range(20):
        kind = trial % 5
        if kind == 0:
            keys = rng.standard_normal(E)
        elif kind == 1:  # heavy ties: few distinct values
            keys = rng.integers(0, 3, E).astype(np.float64)
        elif kind == 2:  # all equal: the order is by id alone
            keys = np.zeros(E)
        elif kind == 3:  # the best keys crowded into one wave
            keys = rng.standard_normal(E)
            keys[: (E + 3) // 4] += 5.0
        else:  # the best keys crowded into one lane of each wave
            keys = rng.standard_normal(E)
            Q = (E + 3) // 4
            for w in range(4):
                keys[w * Q: min(E, (w + 1) * Q): 64] += 10.0
        check(keys, K)


def test_pool_size_at_the_decode_workloads():
    """16 of 896 with sigmoid keys plus a score bias (the decode workload's routing)
    and without it: the pool stays far below the 128-code cap."""
    rng = np.random.default_rng(7)
    sizes = []
    for t in range(400):
        lg = rng.standard_normal(896)
        keys = 1.0 / (1.0 + np.exp(-lg)) + (0.1 * rng.standard_normal(896) if t % 2 else 0.0)
        sizes.append(check(keys, 16))
    assert max(sizes) <= 128, max(sizes)
    assert 16 <= min(sizes)


def _kernel_keys(logits, bias):
    sd = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    key = (sd.astype(np.float32) + bias).astype(np.float32).astype(np.float64)
    key[np.isnan(key)] = -np.inf
    return key


def test_gpu_route_inputs_reach_every_rank_path():
    """The router ranks the pool in wave 0 alone (at most 64 codes), with every wave
    (65..128), or falls back to K rounds of wave maxima (more than 128).  The GPU
    router tests' own inputs (same generators) must reach all three."""
    sizes = []
    for T, E, K in [(3, 100, 7), (5, 64, 64), (2, 4096, 64), (4, 33, 1), (7, 16, 16)]:  # test_route_shapes
        rng = np.random.default_rng(T * 1000 + E)
        logits = rng.standard_normal((T, E)).astype(np.float32)
        bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
        sizes += [len(threshold_pool(_kernel_keys(logits[t], bias), K)) for t in range(T)]
    for E, K in [(896, 16), (4096, 64)]:  # test_route_flat_keys
        rng = np.random.default_rng(E + K)
        logits = np.zeros((3, E), np.float32)
        logits[1] = rng.integers(0, 2, E).astype(np.float32)
        bias = np.zeros(E, np.float32)
        sizes += [len(threshold_pool(_kernel_keys(logits[t], bias), K)) for t in range(3)]
    sizes = np.array(sizes)
    assert np.any(sizes <= 64) and np.any((sizes > 64) & (sizes <= 128)) and np.any(sizes > 128), sizes
