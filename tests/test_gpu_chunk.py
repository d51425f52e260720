"""Chunk path (grouped bf16-MFMA GEMMs) on the GPU vs the oracle: rel-L2 <= 5e-3.

The chunk path takes bf16 activations (both sides see the same bf16 values) and
rounds h to bf16 between the two products (relative error <= 2^-9 per element);
on these weights that alone gives ~1.2e-3, inside the 5e-3 budget (the pages
measure 3.5e-3 for per-32 int8 activations)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _chunk_gpu(W, x, idx, w):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    xb = torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)  # exact: x holds bf16 values
    assert np.array_equal(xb.float().cpu().numpy(), x)
    y = lib.forward_chunk(W, xb, torch.from_numpy(np.ascontiguousarray(idx)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(w)).cuda(), n_unique=nu)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(nu.item())


def _full_case(cfg, what, T=None):
    x, logits, bias = synth.activations(cfg, T=T)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    log(f"chunk {what}: T={x.shape[0]} E={cfg.E} K={cfg.K} D={cfg.D} F={cfg.F}")
    got, nu = _chunk_gpu(W, x, idx, w)
    assert nu == len(np.unique(idx))
    log(f"chunk {what}: union {nu}, dedup {idx.size / nu:.2f}x; running oracle")
    want = oracle_forward_subset(cfg, x, idx, w)
    assert_close(got, want, TOL, f"chunk {what}")
    return got, x, idx, w


def test_chunk_tiny_ragged():
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=5, path="chunk")
    _full_case(cfg, "tiny T=5")


@pytest.mark.parametrize("E,K,D,F,T", [(8, 4, 512, 384, 600), (16, 4, 352, 160, 100), (6, 6, 256, 128, 131)])
def test_chunk_tiles_and_tails(E, K, D, F, T):
    """Several tiles per expert, a ragged last tile, and widths that are not
    multiples of the 128-wide steps and column blocks."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name=f"ch{E}_{K}_{D}_{F}", E=E, K=K, D=D, F=F, T=T,
                       weight_seed=800 + E, act_seed=800 + T, path="chunk")
    _full_case(cfg, f"E={E} K={K} D={D} F={F} T={T}")


def test_chunk_prefill32():
    _full_case(synth.CONFIGS["prefill32"], "prefill32")


def test_chunk_prefill256():
    _full_case(synth.CONFIGS["prefill256"], "prefill256")


def test_chunk_batch4096_sampled():
    """Full 4096-token launch; the oracle checks a seeded sample of tokens plus a
    sample of the tokens routed to the full-scale-range edge experts."""
    cfg = synth.CONFIGS["batch4096"]
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    log("chunk batch4096: GPU run")
    got, nu = _chunk_gpu(W, x, idx, w)
    assert nu == len(np.unique(idx))
    edge_tok = np.nonzero(np.isin(idx, cfg.edge_experts).any(axis=1))[0]
    rng = np.random.default_rng(42)
    pick_edge = rng.choice(edge_tok, size=min(48, len(edge_tok)), replace=False)
    sample = synth.sample_tokens(cfg, 64, must_include=pick_edge, seed=1)
    log(f"chunk batch4096: union {nu}; {len(edge_tok)} edge-expert tokens; oracle on {len(sample)} tokens")
    want = oracle_forward_subset(cfg, x[sample], idx[sample], w[sample])
    assert_close(got[sample], want, TOL, "chunk batch4096 sample")
    # tokens that avoid the edge experts must come out finite
    fin = np.isfinite(got).all(axis=1)
    normal = np.setdiff1d(np.arange(cfg.T), edge_tok)
    assert fin[normal].all()
    log(f"chunk batch4096: finite tokens {int(fin.sum())} / {cfg.T}")


def test_chunk_matches_decode_per_token():
    """GPU self-consistency: the chunk path agrees with the fp32 decode path."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["prefill32"]
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    got, _ = _chunk_gpu(W, x, idx, w)
    for t in (0, 7, 31):
        y = lib.forward_decode(W, torch.from_numpy(x[t]).cuda(), torch.from_numpy(idx[t]).cuda(),
                               torch.from_numpy(w[t]).cuda()).cpu().numpy()
        assert_close(got[t], y, TOL, f"chunk vs decode token {t}")


def test_chunk_deterministic_and_invalid():
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=70, path="chunk")
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    a, _ = _chunk_gpu(W, x, idx, w)
    b, _ = _chunk_gpu(W, x, idx, w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    bad = idx.copy()
    bad[5, 1] = bad[5, 0]
    y, nu = _chunk_gpu(W, x, bad, w)
    assert nu == -1 and np.all(np.isnan(y))
