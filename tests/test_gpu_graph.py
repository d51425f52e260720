"""The decode path, the chunk path and the LatentMoE block replayed from a HIP graph
(torch.cuda.CUDAGraph around the same library calls, as the benchmark times
them): every replay, with eager work and synchronizations between replays, must
reproduce the eager outputs bit for bit."""
import numpy as np
import pytest

import synth
from gpu_helpers import device_weights, log, torch_cuda

pytestmark = pytest.mark.gpu


def _capture(torch, fn, n):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["tiny", "decode1"])
def test_decode_graph_replays_equal_eager(name):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS[name]
    W = device_weights(cfg)
    n = 4
    xs, logits, bias = synth.activations(cfg, T=n, stream=41)
    x_d, l_d, b_d = (torch.from_numpy(a).cuda() for a in (xs, logits, bias))
    idx = torch.empty((n, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, cfg.K), dtype=torch.float32, device="cuda")
    y = torch.empty((n, cfg.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.workspace_size(lib.OP_DECODE, 1, cfg.K, W), dtype=torch.uint8, device="cuda")

    def step(j):
        lib.route(l_d[j:j + 1], b_d, cfg.K, idx=idx[j:j + 1], w=w[j:j + 1])
        lib.forward_decode(W, x_d[j], idx[j], w[j], y=y[j], ws=ws)

    for j in range(n):
        step(j)
    torch.cuda.synchronize()
    want = y.clone()
    g = _capture(torch, step, n)
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), f"{name}: replay {rep} differs"
        # eager work between replays, on other data
        lib.forward_decode(W, x_d[(rep + 1) % n], idx[0], w[0], y=y[0], ws=ws)
        torch.cuda.synchronize()
    log(f"decode graph ({name}): 3 replays of {n} steps equal the eager outputs")
    del g


def test_latent_one_token_graph_replays_equal_eager():
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent_tiny"]
    cfg = lc.experts
    W = device_weights(cfg)
    dh = synth.latent_dense_host(lc)
    L = lib.LatentWeights({k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in dh.items()}, lc.eps)
    n = 3
    h, lg, b = synth.latent_activations(lc, T=n)
    h_d = torch.from_numpy(h).to(torch.bfloat16).cuda()
    idx, w = lib.route(torch.from_numpy(lg).cuda(), torch.from_numpy(b).cuda(), cfg.K)
    out = torch.empty((n, lc.Dh), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.load().k3moe_latent_workspace_size(L.ref(), 1, cfg.K, W.ref()), dtype=torch.uint8,
                     device="cuda")

    def step(j):
        lib.latent_forward(L, W, h_d[j:j + 1], idx[j:j + 1], w[j:j + 1], out=out[j:j + 1], ws=ws)

    for j in range(n):
        step(j)
    torch.cuda.synchronize()
    want = out.clone()
    g = _capture(torch, step, n)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"latent replay {rep} differs"
        step((rep + 1) % n)  # eager work between replays
        torch.cuda.synchronize()
    assert np.all(np.isfinite(want.cpu().numpy()))
    log("latent one-token graph: 3 replays equal the eager outputs")
    del g


def _replays_equal(torch, fn, outs, n_rep=3, what=""):
    """Capture fn() once; each replay (outputs poisoned first, eager work on other data
    between replays) must reproduce the eager outputs bit for bit."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = _capture(torch, lambda i: fn(), 1)
    for rep in range(n_rep):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, wnt in zip(outs, want):
            assert torch.equal(o.view(torch.int32), wnt.view(torch.int32)), f"{what}: replay {rep} differs"
        fn(eager_other=True)
        torch.cuda.synchronize()
    del g
    return want


def test_chunk_graph_replays_equal_eager():
    """The fp32 chunk path at K3 shape (group, split of x, fp16 / bf16 GEMM items,
    combine) replayed from a graph: no memset or host-side state in the capture."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["prefill32"]
    W = device_weights(cfg)
    x, lg, b = synth.activations(cfg)
    x_d = torch.from_numpy(x).cuda()
    x_other = torch.flip(x_d, dims=[0]).contiguous()
    idx, w = lib.route(torch.from_numpy(lg).cuda(), torch.from_numpy(b).cuda(), cfg.K)
    y = torch.empty((x.shape[0], cfg.D), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    ws = torch.empty(lib.workspace_size(lib.OP_CHUNK, x.shape[0], cfg.K, W), dtype=torch.uint8, device="cuda")

    def fn(eager_other=False):
        if eager_other:
            lib.forward_chunk(W, x_other, idx, w, y=y2, ws=ws)
        else:
            lib.forward_chunk(W, x_d, idx, w, y=y, ws=ws)

    want = _replays_equal(torch, fn, [y], what="chunk")
    assert np.all(np.isfinite(want[0].cpu().numpy()))
    log("chunk graph (prefill32, fp32 x): 3 replays equal the eager output")


def test_latent_chunk_graph_replays_equal_eager():
    """The LatentMoE block for 32 tokens at K3 shape (dense MFMA products with split
    reductions whose counters the block clears itself, the routed chunk path, RMSNorm)
    replayed from a graph."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    lc = synth.LATENT["latent32"]
    cfg = lc.experts
    W = device_weights(cfg)
    dh = synth.latent_dense_host(lc)
    L = lib.LatentWeights({k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in dh.items()}, lc.eps)
    h, lg, b = synth.latent_activations(lc)
    T = h.shape[0]
    h_d = torch.from_numpy(h).to(torch.bfloat16).cuda()
    h_other = torch.flip(h_d, dims=[0]).contiguous()
    idx, w = lib.route(torch.from_numpy(lg).cuda(), torch.from_numpy(b).cuda(), cfg.K)
    out = torch.empty((T, lc.Dh), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    ws = torch.empty(lib.load().k3moe_latent_workspace_size(L.ref(), T, cfg.K, W.ref()), dtype=torch.uint8,
                     device="cuda")

    def fn(eager_other=False):
        if eager_other:
            lib.latent_forward(L, W, h_other, idx, w, out=out2, ws=ws)
        else:
            lib.latent_forward(L, W, h_d, idx, w, out=out, ws=ws)

    want = _replays_equal(torch, fn, [out], what="latent chunk")
    assert np.all(np.isfinite(want[0].cpu().numpy()))
    log(f"latent chunk graph (T={T}, K3 shape): 3 replays equal the eager output")
