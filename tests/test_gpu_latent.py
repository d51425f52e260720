"""LatentMoE block (projections, routed experts, RMSNorm, shared experts) on the GPU
vs the oracle: rel-L2 <= 5e-3.

The GPU runs the dense products as bf16 x bf16 with fp32 accumulation, keeps the
latent input x in fp32 (as the oracle does: nothing is rounded between the
projection and the experts), and rounds the normed aggregate and the shared
experts' activation to bf16 (2^-9 relative each); the routed block adds its own
error (decode: fp32-accurate; chunk: see the chunk tests).  The oracle keeps
every sum in double."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 5e-3
_dense_cache = {}


def _dense_device(lc):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    if lc.name not in _dense_cache:
        _dense_cache.clear()
        host = synth.latent_dense_host(lc)
        dev = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in host.items()}  # exact: bf16 values
        _dense_cache[lc.name] = (host, lib.LatentWeights(dev, lc.eps))
    return _dense_cache[lc.name]


def _run(lc, T=None, what=""):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = lc.experts
    host, L = _dense_device(lc)
    W = device_weights(cfg)
    h, logits, bias = synth.latent_activations(lc, T=T)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    log(f"latent {what}: T={h.shape[0]} Dh={lc.Dh} Dl={cfg.D} Fs={lc.Fs} E={cfg.E} K={cfg.K}")
    out = lib.latent_forward(L, W, torch.from_numpy(h).to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    used = np.unique(idx)
    Wh = synth.weights_host(cfg, used)
    local = np.searchsorted(used, idx).astype(np.int32)
    dense = {"w_dn": host["w_down"], "w_up": host["w_up"], "norm": host["norm"], "eps": lc.eps,
             "sg": host["shared_gate"], "su": host["shared_up"], "sd": host["shared_down"]}
    want = oracle.latent_forward(dense, Wh, h, local, w)
    assert_close(got, want, TOL, f"latent {what}")
    return got


def test_latent_tiny_chunk():
    _run(synth.LATENT["latent_tiny"], what="tiny T=6 (chunk path)")


def test_latent_tiny_one_token():
    _run(synth.LATENT["latent_tiny"], T=1, what="tiny T=1 (decode path)")


def test_latent_k3_one_token():
    _run(synth.LATENT["latent1"], what="K3 shape, 1 token")


def test_latent_k3_32_tokens():
    _run(synth.LATENT["latent32"], what="K3 shape, 32 tokens")


def test_latent_deterministic():
    a = _run(synth.LATENT["latent_tiny"], what="tiny repeat a")
    b = _run(synth.LATENT["latent_tiny"], what="tiny repeat b")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("T", [2, 5, 70, 300])
def test_latent_ragged_token_counts(T):
    """Token counts that are not multiples of the 64-token grouping block; 300 spans
    three 128-row token tiles of the dense products, the last one ragged."""
    _run(synth.LATENT["latent_tiny"], T=T, what=f"tiny T={T}")


def test_latent_latent_width_not_multiple_of_64():
    """A latent width of 288 (the routed experts' d_model): the out product's first
    segment (W_up r) ends half-way through a step and the second (S_d s) starts on a
    fresh one."""
    import dataclasses
    base = synth.LATENT["latent_tiny"]
    lc = dataclasses.replace(base, name="latent_tiny_288", experts=synth.scaled(base.experts, D=288), Dh=544, Fs=288)
    _run(lc, T=40, what="tiny Dl=288 Dh=544 Fs=288 T=40")
    _run(lc, T=1, what="tiny Dl=288 Dh=544 Fs=288 T=1")


def test_latent_widths_not_multiple_of_64():
    """Hidden width 544 and shared width 288: reductions that end half-way through
    a 64-column step and output widths that end inside a column tile."""
    import dataclasses
    lc = dataclasses.replace(synth.LATENT["latent_tiny"], name="latent_tiny_544", Dh=544, Fs=288)
    _run(lc, T=40, what="tiny Dh=544 Fs=288 T=40")


def test_latent_k3_256_tokens_sampled():
    """The 256-token block at K3 shape, in the configuration the benchmark times (the
    decode1 experts, 128-row token tiles, split reductions), checked on 24 sampled
    tokens: every output token depends only on its own inputs."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent1"]
    cfg = lc.experts
    host, L = _dense_device(lc)
    W = device_weights(cfg)
    h, logits, bias = synth.latent_activations(lc, T=256)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    log(f"latent K3 256 tokens: T=256 Dh={lc.Dh} Dl={cfg.D} Fs={lc.Fs}")
    out = lib.latent_forward(L, W, torch.from_numpy(h).to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    s = np.random.default_rng(256).choice(256, 24, replace=False)
    s.sort()
    used = np.unique(idx[s])
    Wh = synth.weights_host(cfg, used)
    local = np.searchsorted(used, idx[s]).astype(np.int32)
    dense = {"w_dn": host["w_down"], "w_up": host["w_up"], "norm": host["norm"], "eps": lc.eps,
             "sg": host["shared_gate"], "su": host["shared_up"], "sd": host["shared_down"]}
    want = oracle.latent_forward(dense, Wh, h[s], local, w[s])
    assert_close(got[s], want, TOL, "latent K3 256 tokens (24 sampled)")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("T", [1, 40])
def test_latent_max_widths(T):
    """Hidden and shared widths at the largest supported 8192: the one-token GEMV
    kernels and the chunk's dense MFMA products (reductions of 8192 and of 256 + 8192)."""
    import dataclasses
    lc = dataclasses.replace(synth.LATENT["latent_tiny"], name="latent_tiny_8192", Dh=8192, Fs=8192)
    _run(lc, T=T, what=f"tiny Dh=Fs=8192 T={T}")


def test_latent_k3_chunk_deterministic():
    """Split reductions of the K3-shaped dense products are summed in split order:
    two runs give the same bits whichever split of a tile finishes last."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent32"]
    cfg = lc.experts
    _, L = _dense_device(lc)
    W = device_weights(cfg)
    h, logits, bias = synth.latent_activations(lc, T=64)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    args = (L, W, torch.from_numpy(h).to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(),
            torch.from_numpy(w).cuda())
    a = lib.latent_forward(*args).cpu().numpy()
    b = lib.latent_forward(*args).cpu().numpy()
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_latent_single_expert_per_token():
    import dataclasses
    lc = synth.LATENT["latent_tiny"]
    lc1 = dataclasses.replace(lc, name="latent_tiny_k1", experts=synth.scaled(lc.experts, K=1))
    _run(lc1, what="tiny K=1")
    _run(lc1, T=1, what="tiny K=1, one token")


@pytest.mark.parametrize("T", [1, 6])
def test_latent_every_slot_pruned(T):
    """With every routing slot pruned the routed aggregate is 0, RMSNorm(0) = 0, and the
    block's output is the shared experts alone (against the oracle, which skips the
    pruned slots the same way)."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent_tiny"]
    cfg = lc.experts
    host, L = _dense_device(lc)
    W = device_weights(cfg)
    h, logits, bias = synth.latent_activations(lc, T=T)
    idx = np.full((T, cfg.K), -1, dtype=np.int32)
    w = np.zeros((T, cfg.K), dtype=np.float32)
    out = lib.latent_forward(L, W, torch.from_numpy(h).to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    Wh = synth.weights_host(cfg, np.array([0]))
    dense = {"w_dn": host["w_down"], "w_up": host["w_up"], "norm": host["norm"], "eps": lc.eps,
             "sg": host["shared_gate"], "su": host["shared_up"], "sd": host["shared_down"]}
    want = oracle.latent_forward(dense, Wh, h, idx, w)
    assert_close(got, want, TOL, f"latent every slot pruned T={T}")


@pytest.mark.parametrize("T", [1, 6])
def test_latent_invalid_routing_is_nan(T):
    """An expert id out of range makes the routed block's output NaN (decode: the
    token's row; chunk: the whole chunk, n_unique = -1), and the block's output with it."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent_tiny"]
    cfg = lc.experts
    _, L = _dense_device(lc)
    W = device_weights(cfg)
    h, logits, bias = synth.latent_activations(lc, T=T)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    idx[0, 0] = cfg.E + 3
    out = lib.latent_forward(L, W, torch.from_numpy(h).to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert np.isnan(out.cpu().numpy()[0]).all()
