"""Decode (one token, fp32 path) on the GPU vs the oracle: rel-L2 <= 1e-5.

The tolerance is the fp32-accumulate bound: a 3584-term fp32 sum carries about
u*sqrt(n/2) ~ 2.5e-6 relative error per stage, and the oracle sums in double."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, timing_event, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _decode_gpu(W, x, idx, w):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    y = lib.forward_decode(W, torch.from_numpy(x).cuda(), torch.from_numpy(idx).cuda(),
                           torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _case(cfg, x, logits, bias, what):
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    for t in range(x.shape[0]):
        log(f"decode {what} token {t}: experts {idx[t].tolist()}")
        got = _decode_gpu(W, x[t], idx[t], w[t])
        want = oracle_forward_subset(cfg, x[t:t + 1], idx[t:t + 1], w[t:t + 1])[0]
        assert_close(got, want, TOL, f"decode {what} token {t}")


def test_decode_tiny():
    cfg = synth.CONFIGS["tiny"]
    x, logits, bias = synth.activations(cfg, T=4, stream=3)
    _case(cfg, x, logits, bias, "tiny")


def test_decode_k3_shape():
    cfg = synth.CONFIGS["decode1"]
    x, logits, bias = synth.activations(cfg)
    _case(cfg, x, logits, bias, "decode1")
    x2, l2, b2 = synth.activations(cfg, T=2, stream=11)
    _case(cfg, x2, l2, b2, "decode1 extra")


@pytest.mark.parametrize("E,K,D,F", [(5, 3, 352, 160), (64, 64, 64, 96), (4, 1, 8192, 8192), (9, 4, 4160, 2080)])
def test_decode_shapes(E, K, D, F):
    cfg = synth.scaled(synth.CONFIGS["tiny"], name=f"dec{E}_{K}_{D}_{F}", E=E, K=K, D=D, F=F,
                       weight_seed=700 + E, act_seed=700 + K)
    x, logits, bias = synth.activations(cfg, T=1)
    _case(cfg, x, logits, bias, f"E={E} K={K} D={D} F={F}")


def test_decode_edge_scales():
    """An expert whose scale bytes span 0..255: per-weight semantics (inf weights,
    NaN from inf - inf) must match the oracle's non-finite pattern."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name="dec_edge", E=8, K=2, D=256, F=128,
                       weight_seed=901, edge_experts=(1,))
    x, logits, bias = synth.activations(cfg, T=1)
    idx = np.array([[1, 4]], np.int32)
    w = np.array([[0.5, 0.5]], np.float32)
    W = device_weights(cfg)
    got = _decode_gpu(W, x[0], idx[0], w[0])
    want = oracle_forward_subset(cfg, x, idx, w)[0]
    assert_close(got, want, TOL, "decode edge scales")


def test_decode_deterministic_and_invalid_index():
    torch = torch_cuda()
    cfg = synth.CONFIGS["tiny"]
    W = device_weights(cfg)
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    a = _decode_gpu(W, x[0], idx[0], w[0])
    b = _decode_gpu(W, x[0], idx[0], w[0])
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    bad = idx[0].copy()
    bad[1] = cfg.E + 3
    y = _decode_gpu(W, x[0], bad, w[0])
    assert np.all(np.isnan(y))
    # every slot pruned: y = 0 (the combine of no slot)
    y = _decode_gpu(W, x[0], np.full_like(idx[0], -1), w[0])
    assert np.all(y == 0.0)
    del torch


def test_decode_workspace_garbage_and_reuse():
    """The down kernel's combine counters live in the workspace: a workspace full of
    garbage, and one reused by consecutive calls (tokens with different kept-slot
    counts), give the same bits as fresh workspaces."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    W = device_weights(cfg)
    x, logits, bias = synth.activations(cfg, T=3, stream=22)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    idx[1, 3] = -1  # a token with a pruned slot between two full ones
    w[1, 3] = 0.0
    ws = torch.empty(lib.workspace_size(lib.OP_DECODE, 1, cfg.K, W), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    for t in range(3):
        xd, idd, wd = (torch.from_numpy(np.ascontiguousarray(a[t])).cuda() for a in (x, idx, w))
        got = lib.forward_decode(W, xd, idd, wd, ws=ws)
        fresh = lib.forward_decode(W, xd, idd, wd)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint32), fresh.cpu().numpy().view(np.uint32)), t
        want = oracle_forward_subset(cfg, x[t:t + 1], idx[t:t + 1], w[t:t + 1])[0]
        assert_close(got.cpu().numpy(), want, TOL, f"decode reused workspace token {t}")


def test_decode_stages_match_oracle():
    """Stage-wise: h from the gate/up stage vs the oracle's SiTU-GLU activations, and
    the down stage fed with the oracle's own h."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    cfg = synth.CONFIGS["decode1"]
    x, logits, bias = synth.activations(cfg, T=1, stream=21)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    log(f"decode stages: experts {idx[0].tolist()}")
    h = lib.decode_gateup(W, torch.from_numpy(x[0]).cuda(), torch.from_numpy(idx[0]).cuda()).cpu().numpy()
    y_o, ytk, hk = oracle_forward_subset(cfg, x, idx, w, want_pairs=True)
    assert_close(h, hk[0], TOL, "decode stage gate/up h")
    y = lib.decode_down(W, torch.from_numpy(hk[0].astype(np.float32)).cuda(), torch.from_numpy(idx[0]).cuda(),
                        torch.from_numpy(w[0]).cuda()).cpu().numpy()
    want = (w[0].astype(np.float64)[:, None] * ytk[0]).sum(axis=0)
    assert_close(y, want, TOL, "decode stage down (oracle h in)")
    # the stages chained equal the product path bit for bit, and so does the timed
    # product path (gate/up launched with events its launch records)
    xd, idd, wd = torch.from_numpy(x[0]).cuda(), torch.from_numpy(idx[0]).cuda(), torch.from_numpy(w[0]).cuda()
    y_st = lib.decode_down(W, lib.decode_gateup(W, xd, idd), idd, wd)
    y_fw = lib.forward_decode(W, xd, idd, wd)
    ev0, ev1 = timing_event(), timing_event()
    y_t = lib.forward_decode_timed(W, xd, idd, wd, ev0.cuda_event, ev1.cuda_event)
    torch.cuda.synchronize()
    bits = y_fw.cpu().numpy().view(np.uint32)
    assert np.array_equal(y_st.cpu().numpy().view(np.uint32), bits)
    assert np.array_equal(y_t.cpu().numpy().view(np.uint32), bits)
    ms = ev0.elapsed_time(ev1)
    log(f"decode gate/up kernel (own events): {ms * 1e3:.1f} us")
    assert 0.0 < ms < 100.0
