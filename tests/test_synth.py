"""The seeded generator: determinism, per-expert independence, stated ranges."""
import hashlib

import numpy as np

import synth


def test_configs_shapes():
    c = synth.CONFIGS["decode1"]
    assert (c.E, c.K, c.D, c.F) == (896, 16, 3584, 3072)
    assert c.expert_bytes() == 17_547_264                  # ~17.5 MB per expert
    assert 16 * c.expert_bytes() * 92 / 1e9 > 25.8          # 25.8 GB per token over 92 layers
    assert synth.CONFIGS["batch4096"].edge_experts == tuple(range(0, 896, 112))


def test_deterministic_and_independent():
    cfg = synth.CONFIGS["tiny"]
    a = synth.weights_host(cfg)
    b = synth.weights_host(cfg)
    for n in synth.TENSORS:
        assert np.array_equal(a[n], b[n])
    sub = synth.weights_host(cfg, [5, 2])
    for n in synth.TENSORS:
        assert np.array_equal(sub[n][0], a[n][5]) and np.array_equal(sub[n][1], a[n][2])
    h = hashlib.sha256(b"".join(a[n].tobytes() for n in synth.TENSORS)).hexdigest()
    assert h == hashlib.sha256(b"".join(b[n].tobytes() for n in synth.TENSORS)).hexdigest()


def test_ranges():
    cfg = synth.CONFIGS["tiny"]
    W = synth.weights_host(cfg)
    for n in ("gate_s", "up_s", "down_s"):
        assert W[n].min() >= 120 and W[n].max() <= 130
    lo = W["gate_q"] & 0xF
    hi = W["gate_q"] >> 4
    assert set(np.unique(lo)) == set(range(16)) and set(np.unique(hi)) == set(range(16))
    big = synth.CONFIGS["batch4096"]
    normal = synth.expert_tensors(big, 1)
    assert normal["gate_s"].min() == 118 and normal["gate_s"].max() == 128


def test_activations():
    cfg = synth.CONFIGS["prefill32"]
    x, logits, bias = synth.activations(cfg)
    assert x.shape == (32, 3584) and x.dtype == np.float32
    assert logits.shape == (32, 896) and np.all(bias == 0)
    assert abs(float(np.std(logits)) - 1.0) < 0.05          # h.R with var(R) = 1/D
    assert abs(float(np.std(x)) - 1.0) < 0.05                # stationary AR(1)
    corr = float(np.mean(x[1:] * x[:-1]))
    assert abs(corr - 0.9) < 0.05                            # lag-1 correlation 0.9
    c1 = synth.CONFIGS["tiny"]
    x1, l1, b1 = synth.activations(c1)
    assert x1.shape == (1, 256) and l1.shape == (1, 8) and b1.shape == (8,) and np.any(b1 != 0)
    xa, _, _ = synth.activations(c1, T=4, stream=1)
    xb, _, _ = synth.activations(c1, T=4, stream=2)
    assert not np.array_equal(xa, xb)


def test_activation_precision():
    """Hidden states are fp32 except for the workload that names bf16 activations
    (prefill256), whose values are bf16 held in fp32."""
    for name, is_bf16 in (("prefill32", False), ("batch4096", False), ("decode1", False), ("prefill256", True)):
        x, _, _ = synth.activations(synth.CONFIGS[name], T=8)
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0) == is_bf16, name
    # round to nearest, ties to even
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], np.float32)
    assert synth.bf16_round(v).tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0]


def test_edge_experts():
    """Edge experts of the 4096-token workload: every scale byte 0..255 and every code
    occur; groups above 128 hold only +-0 codes; about a quarter of the groups carry
    an edge scale; the literal mode draws all scale bytes over 0..255."""
    big = synth.CONFIGS["batch4096"]
    edge = synth.expert_tensors(big, 112)
    for t in ("gate", "up", "down"):
        q, sc = edge[t + "_q"], edge[t + "_s"]
        assert set(np.unique(sc)) == set(range(256))
        codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1, 32)
        assert set(np.unique(codes)) == set(range(16))
        high = sc > synth.EDGE_ZERO_ABOVE
        assert np.all(np.isin(codes[high], (0, 8)))
        frac = np.mean((sc < big.scale_lo) | (sc > big.scale_hi))
        assert 0.2 < frac < 0.25
    lit = synth.expert_tensors(synth.scaled(big, edge_mode="literal"), 112)
    assert np.mean((lit["gate_s"] < 118) | (lit["gate_s"] > 128)) > 0.9
