"""MXFP4 decode on the GPU vs the oracle, bit for bit (fp32 and bf16 outputs)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import log, torch_cuda

pytestmark = pytest.mark.gpu


def _bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _run(q, s):
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    qd = torch.from_numpy(q).cuda()
    sd = torch.from_numpy(s).cuda()
    f32 = lib.dequant_mxfp4(qd, sd, torch.float32).cpu().numpy()
    bf = lib.dequant_mxfp4(qd, sd, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    torch.cuda.synchronize()
    return f32, bf


def _check(q, s, what):
    want = _bits32(oracle.dequant(q, s))
    f32, bf = _run(q, s)
    got = _bits32(f32)
    n32 = int(np.count_nonzero(got != want))
    # every decoded value has its low 16 bits zero, so bf16 is the high half exactly
    assert np.all((want & 0xFFFF) == 0)
    nbf = int(np.count_nonzero(bf.astype(np.uint32) != (want >> 16)))
    log(f"dequant {what} {q.shape}: f32 mismatches {n32}, bf16 mismatches {nbf}")
    assert n32 == 0 and nbf == 0


def test_all_codes_all_scales():
    """16 codes x 256 scale bytes: row s holds every code at scale byte s."""
    q = np.zeros((256, 16), np.uint8)
    for s in range(256):
        for j in range(16):  # byte j = codes (2j % 16, (2j+1) % 16) -> all 16 codes twice
            q[s, j] = ((2 * j) % 16) | ((((2 * j) + 1) % 16) << 4)
    s = np.arange(256, dtype=np.uint8).reshape(256, 1)
    _check(q, s, "16x256 table")


def test_random_bytes_full_scale_range():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(300, 160), dtype=np.uint8)
    s = rng.integers(0, 256, size=(300, 10), dtype=np.uint8)
    _check(q, s, "random")


@pytest.mark.parametrize("name,expert,tensor", [("tiny", 3, "gate"), ("decode1", 0, "down"),
                                                ("batch4096", 112, "gate"), ("batch4096", 784, "down")])
def test_config_tensors(name, expert, tensor):
    cfg = synth.CONFIGS[name]
    ex = synth.expert_tensors(cfg, expert)
    _check(ex[tensor + "_q"], ex[tensor + "_s"], f"{name} expert {expert} {tensor}")
