"""Chunk path (grouped MFMA GEMMs) on the GPU vs the oracle: rel-L2 <= 5e-3.

fp32 activations (the 32- and 4096-token workloads) go through
k3moe_forward_chunk: a work item whose weights are all fp16 normals runs on the
fp16 MFMA with x and h rounded to fp16 (CPU emulation at the K3 shape: 9.4e-4 from
the exact block); other items (scale bytes outside 114..140, byte 255, ragged
steps, or some |x| past the fp16 range) take x = bf16(x) + lo, the low part as
MXFP4 in a second product into the same accumulators (1.5e-3), with h converted
to bf16 for their down products.  Rounding x to bf16 alone would cost 7.3e-3, over
the budget: test_chunk_prefill32 checks the fp32 path against that.  The
256-token workload has bf16 activations and goes through k3moe_forward_chunk_bf16
with both sides seeing the same bf16 values.

The 4096-token launch is checked on at least 512 seeded tokens plus every token
routed to an edge expert (whose scale bytes span 0..255), each token computed by
the oracle; the global rel-L2 and the largest per-token rel-L2 are both bounded."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_weights, log, oracle_forward_subset, rel_l2, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _chunk_gpu(W, x, idx, w, bf16=False):
    """fp32 x through k3moe_forward_chunk, or (bf16=True, x holding bf16 values)
    through k3moe_forward_chunk_bf16."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    if bf16:
        xd = xd.to(torch.bfloat16)
        assert np.array_equal(xd.float().cpu().numpy(), x)  # exact: x holds bf16 values
    y = lib.forward_chunk(W, xd, torch.from_numpy(np.ascontiguousarray(idx)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(w)).cuda(), n_unique=nu)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(nu.item())


def per_token_max(got, want):
    return max(rel_l2(got[t], want[t]) for t in range(got.shape[0]))


def _full_case(cfg, what, T=None, bf16=None):
    bf16 = cfg.x_bf16 if bf16 is None else bf16
    x, logits, bias = synth.activations(cfg, T=T, bf16=bf16)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    log(f"chunk {what}: T={x.shape[0]} E={cfg.E} K={cfg.K} D={cfg.D} F={cfg.F} x={'bf16' if bf16 else 'fp32'}")
    got, nu = _chunk_gpu(W, x, idx, w, bf16=bf16)
    assert nu == len(np.unique(idx))
    log(f"chunk {what}: union {nu}, dedup {idx.size / nu:.2f}x; running oracle")
    want = oracle_forward_subset(cfg, x, idx, w)
    e = assert_close(got, want, TOL, f"chunk {what}")
    pt = per_token_max(got, want)
    log(f"chunk {what}: largest per-token rel-L2 {pt:.3e}")
    assert pt <= TOL
    return got, x, idx, w, e


def test_chunk_tiny_ragged():
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=5, path="chunk")
    _full_case(cfg, "tiny T=5")


def test_chunk_one_token():
    """A chunk of one token: one pair per touched expert, 16-row tiles."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=1, path="chunk")
    _full_case(cfg, "tiny T=1")
    _full_case(cfg, "tiny T=1 bf16 x", bf16=True)


def test_chunk_tiny_bf16_entry():
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=70, path="chunk", x_bf16=True)
    _full_case(cfg, "tiny T=70 bf16 x")


@pytest.mark.parametrize("E,K,D,F,T", [(8, 4, 512, 384, 600), (16, 4, 352, 160, 100), (6, 6, 256, 128, 131),
                                     (64, 64, 256, 128, 20), (4096, 16, 128, 64, 3)])
def test_chunk_tiles_and_tails(E, K, D, F, T):
    """Several tiles per expert, a ragged last tile, and widths that are not
    multiples of the 128-wide steps and column blocks (the low part's rows are
    padded to whole steps)."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name=f"ch{E}_{K}_{D}_{F}", E=E, K=K, D=D, F=F, T=T,
                       weight_seed=800 + E, act_seed=800 + T, path="chunk")
    _full_case(cfg, f"E={E} K={K} D={D} F={F} T={T}")
    _full_case(cfg, f"E={E} K={K} D={D} F={F} T={T}", bf16=True)


@pytest.mark.parametrize("scale_lo,scale_hi", [(120, 130), (100, 113)])
def test_chunk_max_widths(scale_lo, scale_hi):
    """D = F = 8192 (the largest widths) with 24 pairs per expert: 96-row tiles whose
    scale rows for eight waves would not fit in LDS, so the four-wave kernels run;
    scale bytes 120..130 put every item on the fp16 body, 100..113 (below the fp16
    normals) every item on the bf16 + low-part fallback.  A CPU emulation of the two
    roundings on these weights gives 2.3e-3 and 1.7e-3.  (Scale bytes up to 140 make
    8192-term gate sums large enough that the SiTU-GLU transitions amplify either
    rounding of x past the budget: 1.8e-2 for fp16 and for bf16 + low part alike, the
    same in the emulation as on the GPU.)"""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name=f"chmax{scale_lo}", E=4, K=2, D=8192, F=8192, T=48,
                       weight_seed=870 + scale_lo, act_seed=871, scale_lo=scale_lo, scale_hi=scale_hi, path="chunk")
    _full_case(cfg, f"D=F=8192 scales {scale_lo}..{scale_hi}")
    if scale_lo == 120:
        _full_case(cfg, "D=F=8192 bf16 x", bf16=True)


def test_chunk_prefill32():
    """fp32 x: within the budget, and well inside what the bf16 entry reaches on the
    same tokens rounded to bf16 (measured against the exact block on the fp32 x),
    so the low part carries the residual."""
    cfg = synth.CONFIGS["prefill32"]
    got, x, idx, w, e32 = _full_case(cfg, "prefill32")
    W = device_weights(cfg)
    gotb, _ = _chunk_gpu(W, synth.bf16_round(x), idx, w, bf16=True)
    want = oracle_forward_subset(cfg, x, idx, w)
    eb = rel_l2(gotb, want)
    log(f"chunk prefill32: fp32 x {e32:.3e}, x rounded to bf16 {eb:.3e}")
    assert e32 < 0.5 * eb


def test_chunk_prefill256():
    _full_case(synth.CONFIGS["prefill256"], "prefill256")


def test_chunk_batch4096_sampled():
    """The full 4096-token launch (the configuration the benchmark times).  The
    oracle computes 512 seeded tokens plus every token routed to an edge expert;
    masks, global rel-L2 and per-token rel-L2 are checked on all of them, and every
    token's output is finite (the edge experts' weights are finite)."""
    cfg = synth.CONFIGS["batch4096"]
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    log("chunk batch4096: GPU run")
    got, nu = _chunk_gpu(W, x, idx, w)
    assert nu == len(np.unique(idx))
    assert np.isfinite(got).all()
    edge_tok = np.nonzero(np.isin(idx, cfg.edge_experts).any(axis=1))[0]
    sample = synth.sample_tokens(cfg, 512, must_include=edge_tok, seed=1)
    log(f"chunk batch4096: union {nu}; {len(edge_tok)} edge-expert tokens; oracle on {len(sample)} tokens")
    want = oracle_forward_subset(cfg, x[sample], idx[sample], w[sample], progress=128)
    assert_close(got[sample], want, TOL, "chunk batch4096 sample")
    pt = per_token_max(got[sample], want)
    is_edge = np.isin(sample, edge_tok)
    e_edge = rel_l2(got[sample[is_edge]], want[is_edge])
    log(f"chunk batch4096: largest per-token rel-L2 {pt:.3e}; edge tokens alone {e_edge:.3e}")
    assert pt <= TOL and e_edge <= TOL


def test_chunk_x_beyond_fp16():
    """fp32 x with entries past the fp16 range (|x| >= 65520): the launch takes the
    bf16 high part plus MXFP4 low part for every item, and still meets the oracle."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name="x_big", T=40, path="chunk", weight_seed=91, act_seed=91)
    x, logits, bias = synth.activations(cfg)
    x = x.copy()
    x[3, 7] = 7.0e4
    x[17, 100] = -1.0e5
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    got, _ = _chunk_gpu(W, x, idx, w)
    want = oracle_forward_subset(cfg, x, idx, w)
    assert_close(got, want, TOL, "chunk x beyond fp16")
    assert per_token_max(got, want) <= TOL


def test_chunk_literal_edge_masks():
    """Edge experts whose scale bytes are all uniform over 0..255 (weights up to
    +-inf): the non-finite pattern of every output equals the oracle's, and the
    finite outputs agree."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], name="literal_edge", T=60, path="chunk", weight_seed=61,
                       act_seed=61, edge_experts=(1, 5), edge_mode="literal")
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = oracle.route(logits, bias, cfg.K)
    W = device_weights(cfg)
    got, _ = _chunk_gpu(W, x, idx, w)
    want = oracle_forward_subset(cfg, x, idx, w)
    log(f"chunk literal edges: {int((~np.isfinite(want)).any(axis=1).sum())} of {cfg.T} tokens non-finite")
    assert_close(got, want, TOL, "chunk literal edges")


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
    for bf16 in (False, True):
        xx = synth.bf16_round(x) if bf16 else x
        a, _ = _chunk_gpu(W, xx, idx, w, bf16=bf16)
        b, _ = _chunk_gpu(W, xx, idx, w, bf16=bf16)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        bad = idx.copy()
        bad[5, 1] = bad[5, 0]
        y, nu = _chunk_gpu(W, xx, bad, w, bf16=bf16)
        assert nu == -1 and np.all(np.isnan(y))
