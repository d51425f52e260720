"""Top-p pruning on the GPU vs the oracle (colibri PR #676, K3_TOPP paragraph):
kept sets and counts bit-exact, weights to 2 ulp; decode and chunk outputs with
pruned slots within their path's tolerance; grouping skips pruned slots."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, torch_cuda

pytestmark = pytest.mark.gpu


def _route_topp_gpu(logits, bias, K, p):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    idx, w, n = lib.route_topp(torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda(), K, p)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), n.cpu().numpy()


def _compare(logits, bias, K, p, what):
    idx_o, w_o, n_o, gap = oracle.route_topp(logits, bias, K, p)
    idx_g, w_g, n_g = _route_topp_gpu(logits, bias, K, p)
    log(f"topp {what} p={p}: mean kept {n_o.mean():.2f} of {K}")
    assert np.array_equal(n_g, n_o)
    assert np.array_equal(idx_g, idx_o), np.nonzero(np.any(idx_g != idx_o, axis=1))[0][:10]
    kept = idx_o >= 0
    assert np.all(w_g[~kept] == 0.0)
    rel = np.abs(w_g[kept].astype(np.float64) - w_o[kept]) / np.abs(w_o[kept])
    assert rel.max() <= 2 * 2.0 ** -24, rel.max()
    return idx_o, w_o


@pytest.mark.parametrize("name", ["tiny", "decode1", "prefill256"])
@pytest.mark.parametrize("p", [0.3, 0.7, 0.9])
def test_route_topp_configs(name, p):
    cfg = synth.CONFIGS[name]
    _, logits, bias = synth.activations(cfg, T=max(cfg.T, 32) if name != "prefill256" else None, stream=17)
    _compare(logits, bias, cfg.K, p, name)


@pytest.mark.parametrize("p", [0.0, 1.0, 2.0])
def test_route_topp_off_equals_route(p):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    _, logits, bias = synth.activations(cfg, T=16, stream=19)
    idx_g, w_g, n_g = _route_topp_gpu(logits, bias, cfg.K, p)
    i2, w2 = lib.route(torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda(), cfg.K)
    assert np.array_equal(idx_g, i2.cpu().numpy())
    assert np.array_equal(w_g.view(np.uint32), w2.cpu().numpy().view(np.uint32))
    assert np.all(n_g == cfg.K)


@pytest.mark.parametrize("T,E,K", [(9, 64, 64), (5, 4096, 16), (6, 20, 1), (4, 100, 33)])
def test_route_topp_shapes(T, E, K):
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    for p in (0.05, 0.5, 0.95):
        _compare(logits, bias, K, p, f"{T}x{E} K={K}")


def test_decode_topp():
    """One K3-shape token per pruning level through forward_decode (pruned slots skipped)."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    x, logits, bias = synth.activations(cfg, T=2, stream=23)
    W = device_weights(cfg)
    for p in (0.5, 0.8):
        idx, w = _compare(logits, bias, cfg.K, p, "decode1 tokens")
        for t in range(x.shape[0]):
            y = lib.forward_decode(W, torch.from_numpy(x[t]).cuda(), torch.from_numpy(idx[t]).cuda(),
                                   torch.from_numpy(w[t]).cuda())
            torch.cuda.synchronize()
            want = oracle_forward_subset(cfg, x[t:t + 1], idx[t:t + 1], w[t:t + 1])[0]
            assert_close(y.cpu().numpy(), want, 1e-5, f"decode top-p {p} token {t}")


def test_chunk_topp():
    """A 32-token chunk routed with top-p 0.7 through forward_chunk and k3moe_group."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["prefill32"]
    x, logits, bias = synth.activations(cfg)
    idx, w = _compare(logits, bias, cfg.K, 0.7, "prefill32")
    W = device_weights(cfg)
    y = lib.forward_chunk(W, torch.from_numpy(x).cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda())
    g = lib.group(torch.from_numpy(idx).cuda(), cfg.E)
    torch.cuda.synchronize()
    want = oracle_forward_subset(cfg, x, idx, w)
    assert_close(y.cpu().numpy(), want, 5e-3, "chunk top-p 0.7")
    go = oracle.group(idx, cfg.E)
    assert int(g["n_unique"].item()) == go["n_unique"]
    assert np.array_equal(g["counts"].cpu().numpy(), go["counts"])
    assert np.array_equal(g["offsets"].cpu().numpy(), go["offsets"])
    assert np.array_equal(g["perm"].cpu().numpy()[:len(go["perm"])], go["perm"])


@pytest.mark.parametrize("E,K,D,F", [(896, 16, 3584, 3072), (40, 8, 512, 192), (12, 5, 352, 160)])
def test_decode_pruned_anywhere(E, K, D, F):
    """Pruned slots at arbitrary positions (not only the tail): the kept slots are
    served by the 32-row split workgroups when D is a multiple of 256 (first two
    shapes), by the 64-row ones otherwise; both within the decode tolerance.  An
    out-of-range expert beside a pruned slot gives an all-NaN output."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    if D == 3584:
        cfg = synth.CONFIGS["decode1"]
    else:
        cfg = synth.scaled(synth.CONFIGS["tiny"], name=f"prune{E}_{K}_{D}_{F}", E=E, K=K, D=D, F=F,
                           weight_seed=1100 + E, act_seed=1100 + K)
    x, logits, bias = synth.activations(cfg, T=1, stream=31)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    rng = np.random.default_rng(E + K)
    for trial in range(3):
        keep = rng.random(cfg.K) < 0.6
        keep[rng.integers(cfg.K)] = True  # at least one kept
        if keep.all():
            keep[rng.integers(cfg.K)] = False
        idx_t = np.where(keep, idx[0], -1).astype(np.int32)
        w_t = np.where(keep, w[0], 0.0).astype(np.float32)
        log(f"decode pruned {E}x{K} D={D}: kept slots {np.nonzero(keep)[0].tolist()}")
        y = lib.forward_decode(W, torch.from_numpy(x[0]).cuda(), torch.from_numpy(idx_t).cuda(),
                               torch.from_numpy(w_t).cuda())
        torch.cuda.synchronize()
        want = oracle_forward_subset(cfg, x, idx_t[None], w_t[None])[0]
        assert_close(y.cpu().numpy(), want, 1e-5, f"decode pruned {E}x{K} D={D} trial {trial}")
    # an out-of-range expert id in a kept slot, another slot pruned
    bad = idx[0].copy()
    bad[0], bad[cfg.K - 1] = cfg.E + 3, -1
    y = lib.forward_decode(W, torch.from_numpy(x[0]).cuda(), torch.from_numpy(bad).cuda(),
                           torch.from_numpy(w[0]).cuda())
    torch.cuda.synchronize()
    assert np.isnan(y.cpu().numpy()).all()


@pytest.mark.parametrize("entry", ["fp32", "bf16", "mx1", "mx2"])
def test_chunk_pruned_tokens_and_empty_union(entry):
    """Tokens with every slot pruned contribute y = 0 (the combine of no slot), the
    others their kept slots; a chunk whose every slot is pruned has an empty union
    (n_unique 0, no GEMM work item) and y = 0 throughout."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.scaled(synth.CONFIGS["tiny"], name="prune_chunk", E=8, K=2, D=256, F=128, T=70, path="chunk")
    x, logits, bias = synth.activations(cfg, bf16=entry == "bf16")
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    idx = idx.copy()
    w = w.copy()
    idx[:10] = -1  # tokens 0..9: every slot pruned
    w[:10] = 0.0
    idx[10:20, 1] = -1  # tokens 10..19: the second slot pruned, the weights renormalized to the first
    w[10:20, 1] = 0.0
    w[10:20, 0] = 1.0
    W = device_weights(cfg)

    def run(idx_, w_):
        nu = torch.zeros(1, dtype=torch.int32, device="cuda")
        xd = torch.from_numpy(x).cuda()
        args = (W, xd.to(torch.bfloat16) if entry == "bf16" else xd, torch.from_numpy(idx_).cuda(),
                torch.from_numpy(w_).cuda())
        if entry.startswith("mx"):
            y = lib.forward_chunk_mx(*args, parts=int(entry[2]), n_unique=nu)
        else:
            y = lib.forward_chunk(*args, n_unique=nu)
        torch.cuda.synchronize()
        return y.cpu().numpy(), int(nu.item())

    got, nu = run(idx, w)
    assert nu == len(np.unique(idx[idx >= 0]))
    assert np.all(got[:10] == 0.0)
    mx = int(entry[2]) if entry.startswith("mx") else 0
    want = oracle_forward_subset(cfg, x, idx, w, mx=mx)
    assert_close(got, want, 5e-3, f"chunk {entry} with pruned tokens")
    empty_idx = np.full_like(idx, -1)
    got0, nu0 = run(empty_idx, np.zeros_like(w))
    assert nu0 == 0
    assert np.all(got0 == 0.0)
    log(f"chunk {entry}: pruned tokens exact zeros, empty union y = 0")
