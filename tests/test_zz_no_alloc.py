"""The allocation-free decode entry point (k3moe_forward_decode_noalloc) on the
GPU, through the C ABI: on the same inputs it must give exactly the output of
k3moe_forward_decode (the same kernels on a caller workspace), on two calls in a
row, the second with a smaller layer (so the fixed scratch keeps the first call's
contents), and both within 1e-5 of the oracle.  Also: a call refused on the host
for a workspace beyond the fixed array, and replays of a graph that captured the
entry point, each equal to the eager result."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _inputs(cfg, T, stream):
    x, logits, bias = synth.activations(cfg, T=T, stream=stream)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    return x, idx, w


def _both(W, x, idx, w):
    """(noalloc output, workspace-entry output) for one token, as numpy."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    xd, id_, wd = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x, idx, w))
    y0 = torch.full((W.D,), float("nan"), dtype=torch.float32, device="cuda")
    lib.forward_decode_noalloc(W, xd, id_, wd, y=y0)
    y1 = lib.forward_decode(W, xd, id_, wd)
    torch.cuda.synchronize()
    return y0.cpu().numpy(), y1.cpu().numpy()


def test_noalloc_matches_decode_two_calls():
    big = synth.CONFIGS["decode1"]
    small = synth.CONFIGS["tiny"]
    Wb, Ws = device_weights(big), device_weights(small)
    xb, ib, wb = _inputs(big, 1, 21)
    xs, is_, ws = _inputs(small, 1, 22)
    log(f"noalloc: call 1 E={big.E} K={big.K} D={big.D} F={big.F}, experts {ib[0].tolist()}")
    a0, a1 = _both(Wb, xb[0], ib[0], wb[0])
    log(f"noalloc: call 2 E={small.E} K={small.K} D={small.D} F={small.F}, experts {is_[0].tolist()}")
    b0, b1 = _both(Ws, xs[0], is_[0], ws[0])
    assert np.array_equal(a0.view(np.uint32), a1.view(np.uint32))
    assert np.array_equal(b0.view(np.uint32), b1.view(np.uint32))
    assert_close(a0, oracle_forward_subset(big, xb, ib, wb)[0], TOL, "noalloc call 1")
    assert_close(b0, oracle_forward_subset(small, xs, is_, ws)[0], TOL, "noalloc call 2")
    # the larger one again after the smaller: stale scratch contents never leak in
    c0, _ = _both(Wb, xb[0], ib[0], wb[0])
    assert np.array_equal(c0.view(np.uint32), a0.view(np.uint32))


def test_noalloc_pruned_slots():
    """A top-p token (pruned slots skip their scratch rows entirely)."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    W = device_weights(cfg)
    x, logits, bias = synth.activations(cfg, T=1, stream=23)
    idx, w, kept, _ = oracle.route_topp(logits, bias, cfg.K, 0.6)
    log(f"noalloc top-p: {int(kept[0])} of {cfg.K} slots kept")
    a0, a1 = _both(W, x[0], idx[0], w[0])
    assert np.array_equal(a0.view(np.uint32), a1.view(np.uint32))
    assert np.isfinite(a0).all()


def test_noalloc_refuses_oversize_on_host():
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.scaled(synth.CONFIGS["tiny"], name="noalloc_big", E=40, K=33, D=8192, F=8192)
    s = lib.WeightsStruct()
    s.n_experts, s.d_model, s.d_ff = cfg.E, cfg.D, cfg.F
    for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        setattr(s, n, 256)
        setattr(s, n + "_stride", 4096)
    p = ctypes.c_void_p(256)
    rc = lib.load().k3moe_forward_decode_noalloc(ctypes.byref(s), p, p, p, cfg.K, p, None)
    assert rc == lib.K3MOE_E_SCRATCH
    torch.cuda.synchronize()


def test_noalloc_graph_replays():
    """Captured once (after an eager call set up the device's scratch address),
    replayed three times with eager work between the replays; every replay equals
    the eager output bit for bit."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    W = device_weights(cfg)
    x, idx, w = _inputs(cfg, 2, 24)
    xd, id_, wd = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x, idx, w))
    want = [lib.forward_decode_noalloc(W, xd[t], id_[t], wd[t]).cpu().numpy() for t in range(2)]
    y = torch.empty((2, cfg.D), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(2):
                lib.forward_decode_noalloc(W, xd[t], id_[t], wd[t], y=y[t], stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        for t in range(2):
            assert np.array_equal(got[t].view(np.uint32), want[t].view(np.uint32)), f"replay {r} token {t}"
        # eager work between replays, on the same scratch
        lib.forward_decode_noalloc(W, xd[1], id_[1], wd[1])
        torch.cuda.synchronize()
    log("noalloc graph: 3 replays equal to the eager outputs")
