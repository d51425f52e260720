"""Chunk grouping (counting sort by expert + union) on the GPU vs the oracle: bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import log, torch_cuda

pytestmark = pytest.mark.gpu


def _group_gpu(idx, E):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    out = lib.group(torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda(), E)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _compare(idx, E, what):
    log(f"group {what}: T={idx.shape[0]} K={idx.shape[1]} E={E}")
    want = oracle.group(idx, E)
    got = _group_gpu(idx, E)
    nu = int(got["n_unique"][0])
    assert nu == want["n_unique"]
    assert np.array_equal(got["counts"], want["counts"])
    assert np.array_equal(got["offsets"], want["offsets"])
    assert np.array_equal(got["perm"][:len(want["perm"])], want["perm"])  # placed pairs only
    assert np.array_equal(got["uniq"][:nu], want["uniq"])
    P = idx.size
    log(f"group {what}: union {nu} experts, dedup {P / max(nu, 1):.2f}x")
    return nu


@pytest.mark.parametrize("name", ["prefill32", "prefill256", "batch4096"])
def test_group_configs(name):
    cfg = synth.CONFIGS[name]
    _, logits, bias = synth.activations(cfg)
    idx, _, _ = oracle.route(logits, bias, cfg.K)
    _compare(idx, cfg.E, name)


@pytest.mark.parametrize("T,K,E", [(1, 16, 896), (65, 16, 896), (100, 3, 7), (129, 64, 64), (300, 2, 4096),
                                   (7, 1, 1)])
def test_group_shapes(T, K, E):
    rng = np.random.default_rng(T + 7 * K + E)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    _compare(idx, E, f"random {T}x{K} E={E}")


def test_group_skewed():
    """Every token routes to the same few experts: counts far above one tile."""
    T, K, E = 700, 4, 50
    idx = np.tile(np.array([3, 17, 0, 49], np.int32), (T, 1))
    nu = _compare(idx, E, "skewed")
    assert nu == 4


@pytest.mark.parametrize("kind", ["out_of_range", "negative", "duplicate"])
def test_group_invalid(kind):
    T, K, E = 70, 4, 32
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    if kind == "out_of_range":
        idx[66, 2] = E
    elif kind == "negative":
        idx[3, 0] = -2  # -1 marks a pruned slot, any other negative is invalid
    else:
        idx[40, 1] = idx[40, 3]
    got = _group_gpu(idx, E)
    assert int(got["n_unique"][0]) == -1
