"""The router on the GPU vs the oracle: indices bit-exact, weights to 2 ulp."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import log, torch_cuda

pytestmark = pytest.mark.gpu


def _route_gpu(logits, bias, K):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    idx, w = lib.route(torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda(), K)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def _compare(logits, bias, K, what):
    idx_o, w_o, gap = oracle.route(logits, bias, K)
    log(f"route {what}: T={logits.shape[0]} E={logits.shape[1]} K={K}")
    idx_g, w_g = _route_gpu(logits, bias, K)
    flagged = int(np.count_nonzero(gap < 1e-6))
    bad = np.nonzero(np.any(idx_g != idx_o, axis=1))[0]
    log(f"route {what}: {len(bad)} token(s) differ, {flagged} near-tie token(s) (gap < 1e-6)")
    assert len(bad) == 0, f"index mismatch at tokens {bad[:10]} (gaps {gap[bad[:10]]})"
    fin = np.isfinite(w_o)
    assert np.array_equal(fin, np.isfinite(w_g))
    rel = np.abs(w_g[fin].astype(np.float64) - w_o[fin]) / np.abs(w_o[fin])
    assert rel.size == 0 or rel.max() <= 2 * 2.0 ** -24, rel.max()
    return flagged


@pytest.mark.parametrize("name", ["tiny", "decode1", "prefill32", "prefill256", "batch4096"])
def test_route_configs(name):
    cfg = synth.CONFIGS[name]
    _, logits, bias = synth.activations(cfg)
    _compare(logits, bias, cfg.K, name)


def test_route_decode_bias_diagnostic():
    """The 4096-token logits with the decode config's N(0, 0.1) score bias."""
    cfg = synth.CONFIGS["batch4096"]
    _, logits, _ = synth.activations(cfg)
    bias = (0.1 * np.random.default_rng([105, 31337]).standard_normal(cfg.E)).astype(np.float32)
    _compare(logits, bias, cfg.K, "batch4096+bias")


@pytest.mark.parametrize("T,E,K", [(3, 100, 7), (5, 64, 64), (2, 4096, 64), (4, 33, 1), (7, 16, 16)])
def test_route_shapes(T, E, K):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    _compare(logits, bias, K, f"shape {T}x{E} K={K}")


def test_route_ties_nan_and_signed_zero():
    E = 70
    logits = np.zeros((4, E), np.float32)
    logits[1, ::3] = np.nan
    logits[2] = -100.0                       # sigmoid rounds to a tiny value; keys tie through the bias
    logits[3, :10] = 5.0
    bias = np.zeros(E, np.float32)
    bias[5] = -0.0
    bias[6] = 0.5
    _compare(logits, bias, 12, "ties/NaN")
    # a key of exactly -0.0 + 0 vs +0: sigmoid(-200) rounds to 0 in fp32, bias -0.0
    logits2 = np.full((1, 8), -200.0, np.float32)
    bias2 = np.array([-0.0, 0.0, -0.0, 0.0, -0.0, 0.0, -0.0, 0.0], np.float32)
    _compare(logits2, bias2, 5, "signed zeros")


@pytest.mark.parametrize("E,K", [(896, 16), (4096, 64)])
def test_route_flat_keys(E, K):
    """Keys tied across most experts, so more than 128 codes reach the threshold and
    the router takes its K-rounds fallback: all logits equal (the order is by id
    alone), two values, and equal logits under a bias that ties in groups."""
    rng = np.random.default_rng(E + K)
    logits = np.zeros((3, E), np.float32)
    logits[1] = rng.integers(0, 2, E).astype(np.float32)
    bias = np.zeros(E, np.float32)
    logits2 = np.full((1, E), 0.25, np.float32)
    bias2 = (0.01 * rng.integers(0, 3, E)).astype(np.float32)
    _compare(logits, bias, K, f"flat keys {E}/{K}")
    _compare(logits2, bias2, K, f"grouped ties {E}/{K}")
