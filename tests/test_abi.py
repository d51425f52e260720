"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from mxfp4_routed_expert_k3moe_amd import lib as k3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(k3moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(k3.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = k3.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (K3MOE_\w+) \(?(-?\d+)\)?", text))
    assert int(consts["K3MOE_OK"]) == k3.K3MOE_OK
    assert int(consts["K3MOE_E_NULL"]) == k3.K3MOE_E_NULL
    assert int(consts["K3MOE_E_DIM"]) == k3.K3MOE_E_DIM
    assert int(consts["K3MOE_E_ALIGN"]) == k3.K3MOE_E_ALIGN
    assert int(consts["K3MOE_E_WORKSPACE"]) == k3.K3MOE_E_WORKSPACE
    assert int(consts["K3MOE_E_DEVICE"]) == k3.K3MOE_E_DEVICE
    assert int(consts["K3MOE_E_HIP"]) == k3.K3MOE_E_HIP
    assert int(consts["K3MOE_E_SCRATCH"]) == k3.K3MOE_E_SCRATCH
    assert re.search(r"#define K3MOE_NOALLOC_SCRATCH_BYTES \(\(2u << 20\) \+ \(64u << 10\)\)", text)
    assert k3.NOALLOC_SCRATCH_BYTES == (2 << 20) + (64 << 10)
    assert int(consts["K3MOE_MAX_K"]) == k3.K3MOE_MAX_K
    assert int(consts["K3MOE_PRUNED"]) == k3.PRUNED
    assert int(consts["K3MOE_OP_DECODE"]) == k3.OP_DECODE
    assert int(consts["K3MOE_OP_CHUNK"]) == k3.OP_CHUNK
    assert int(consts["K3MOE_OP_GROUP"]) == k3.OP_GROUP
    assert int(consts["K3MOE_OP_CHUNK_MX"]) == k3.OP_CHUNK_MX
    assert int(consts["K3MOE_IN_F32"]) == k3.IN_F32 and int(consts["K3MOE_IN_BF16"]) == k3.IN_BF16


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(k3.status_string(code), str)
    assert k3.status_string(0) == "ok"


def _struct(E=896, D=3584, F=3072, ptr=256, stride=None):
    s = k3.WeightsStruct()
    s.n_experts, s.d_model, s.d_ff = E, D, F
    for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        setattr(s, n, ptr)
    for n in ("gate_q", "up_q", "down_q"):
        setattr(s, n + "_stride", F * D // 2 if stride is None else stride)
    for n in ("gate_s", "up_s", "down_s"):
        setattr(s, n + "_stride", F * D // 32)
    return s


def test_workspace_sizes():
    lib = k3.load()
    s = _struct()
    dec = lib.k3moe_workspace_size(k3.OP_DECODE, 1, 16, ctypes.byref(s))
    assert dec >= 16 * 3072 * 4 + 16 * 3584 * 4
    ch = lib.k3moe_workspace_size(k3.OP_CHUNK, 4096, 16, ctypes.byref(s))
    P = 4096 * 16
    assert ch >= P * 3584 * 4 + P * 3072 * 2 + 4096 * 3584 * 2 + 4096 * 28 * (64 + 4)  # + x = hi + lo split
    assert lib.k3moe_workspace_size(k3.OP_GROUP, 4096, 16, ctypes.byref(s)) > 0
    mx = lib.k3moe_workspace_size(k3.OP_CHUNK_MX, 4096, 16, ctypes.byref(s))
    assert mx >= P * 3584 * 4 + 2 * P * 3072 + 2 * 4096 * 3584
    assert lib.k3moe_workspace_size(k3.OP_CHUNK_MX, 4096, 16, ctypes.byref(_struct(D=3584 + 32))) == 0
    assert lib.k3moe_workspace_size(99, 1, 16, ctypes.byref(s)) == 0
    assert lib.k3moe_workspace_size(k3.OP_DECODE, 1, 65, ctypes.byref(s)) == 0
    bad = _struct(D=3583)
    assert lib.k3moe_workspace_size(k3.OP_DECODE, 1, 16, ctypes.byref(bad)) == 0


def test_validation_before_any_device_call():
    """Every bad argument below is rejected on the host (this container has no GPU)."""
    lib = k3.load()
    s = _struct()
    p = ctypes.c_void_p(256)
    assert lib.k3moe_route(None, p, 1, 896, 16, p, p, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_route(p, p, 0, 896, 16, p, p, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_route(p, p, 1, 896, 65, p, p, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_route(p, p, 1, 8, 9, p, p, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_route(p, p, 1, 5000, 16, p, p, None) == k3.K3MOE_E_DIM
    d = ctypes.c_double
    assert lib.k3moe_route_topp(None, p, 1, 896, 16, d(0.7), p, p, None, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_route_topp(p, p, 1, 896, 16, d(float("nan")), p, p, None, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_route_topp(p, p, 1, 8, 9, d(0.7), p, p, None, None) == k3.K3MOE_E_DIM
    ws = 1 << 20
    assert lib.k3moe_forward_decode(None, p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_forward_decode(ctypes.byref(s), None, p, p, 16, p, p, ws, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_forward_decode(ctypes.byref(s), p, p, p, 0, p, p, ws, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_forward_decode(ctypes.byref(_struct(D=100)), p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_forward_decode(ctypes.byref(_struct(F=16384)), p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_forward_decode(ctypes.byref(_struct(ptr=264)), p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_ALIGN
    assert lib.k3moe_forward_decode(ctypes.byref(_struct(stride=8)), p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_ALIGN
    assert lib.k3moe_forward_decode(ctypes.byref(s), ctypes.c_void_p(260), p, p, 16, p, p, ws, None) == k3.K3MOE_E_ALIGN
    for name in ("gate_s", "up_s", "down_s"):
        bad_s = _struct()
        setattr(bad_s, name, 264)
        assert lib.k3moe_forward_decode(ctypes.byref(bad_s), p, p, p, 16, p, p, ws, None) == k3.K3MOE_E_ALIGN
        bad_s = _struct()
        setattr(bad_s, name + "_stride", 3584 * 3072 // 32 + 4)
        assert lib.k3moe_forward_chunk(ctypes.byref(bad_s), p, 32, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_ALIGN
    assert lib.k3moe_forward_decode(ctypes.byref(s), p, p, p, 16, p, p, 100, None) == k3.K3MOE_E_WORKSPACE
    # the allocation-free forward: validation as forward_decode; a call whose
    # workspace would exceed the fixed scratch array is refused on the host
    na = lib.k3moe_forward_decode_noalloc
    assert na(None, p, p, p, 16, p, None) == k3.K3MOE_E_NULL
    assert na(ctypes.byref(s), p, p, None, 16, p, None) == k3.K3MOE_E_NULL
    assert na(ctypes.byref(s), p, p, p, 0, p, None) == k3.K3MOE_E_DIM
    assert na(ctypes.byref(s), p, p, p, 65, p, None) == k3.K3MOE_E_DIM
    assert na(ctypes.byref(s), ctypes.c_void_p(260), p, p, 16, p, None) == k3.K3MOE_E_ALIGN
    big = _struct(E=896, D=8192, F=8192)
    assert lib.k3moe_workspace_size(k3.OP_DECODE, 1, 33, ctypes.byref(big)) > k3.NOALLOC_SCRATCH_BYTES
    assert na(ctypes.byref(big), p, p, p, 33, p, None) == k3.K3MOE_E_SCRATCH
    assert na(ctypes.byref(s), p, p, p, 64, p, None) != k3.K3MOE_E_SCRATCH  # K = 64 at the K3 shape fits
    assert "K3MOE_NOALLOC_SCRATCH_BYTES" in k3.status_string(k3.K3MOE_E_SCRATCH)
    # the timed forward: both events are required, the rest as forward_decode
    t = lib.k3moe_forward_decode_timed
    assert t(ctypes.byref(s), p, p, p, 16, p, p, ws, None, p, None) == k3.K3MOE_E_NULL
    assert t(ctypes.byref(s), p, p, p, 16, p, p, ws, p, None, None) == k3.K3MOE_E_NULL
    assert t(ctypes.byref(s), p, p, p, 0, p, p, ws, p, p, None) == k3.K3MOE_E_DIM
    assert t(ctypes.byref(s), ctypes.c_void_p(260), p, p, 16, p, p, ws, p, p, None) == k3.K3MOE_E_ALIGN
    assert t(ctypes.byref(s), p, p, p, 16, p, p, 100, p, p, None) == k3.K3MOE_E_WORKSPACE
    assert lib.k3moe_forward_chunk(ctypes.byref(s), p, 0, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_forward_chunk(ctypes.byref(s), p, 32, p, p, 16, p, None, p, 100, None) == k3.K3MOE_E_WORKSPACE
    assert lib.k3moe_forward_chunk(ctypes.byref(s), p, 32, p, None, 16, p, None, p, ws, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_forward_chunk(ctypes.byref(s), None, 32, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_forward_chunk(ctypes.byref(s), ctypes.c_void_p(260), 32, p, p, 16, p, None, p, ws,
                                   None) == k3.K3MOE_E_ALIGN
    cb = lib.k3moe_forward_chunk_bf16
    assert cb(ctypes.byref(s), None, 32, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_NULL
    assert cb(ctypes.byref(s), p, 0, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert cb(ctypes.byref(s), p, 32, p, p, 16, p, None, p, 100, None) == k3.K3MOE_E_WORKSPACE
    assert cb(ctypes.byref(s), ctypes.c_void_p(264), 32, p, p, 16, p, None, p, ws, None) == k3.K3MOE_E_ALIGN
    assert lib.k3moe_group(p, 32, 16, 896, p, p, p, p, p, p, 10, None) == k3.K3MOE_E_WORKSPACE
    assert lib.k3moe_group(p, 32, 0, 896, p, p, p, p, p, p, ws, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_group(None, 32, 16, 896, p, p, p, p, p, p, ws, None) == k3.K3MOE_E_NULL
    assert lib.k3moe_dequant_mxfp4(p, p, 4, 48, p, 0, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_dequant_mxfp4(p, p, 4, 64, p, 7, None) == k3.K3MOE_E_DIM
    assert lib.k3moe_dequant_mxfp4(ctypes.c_void_p(257), p, 4, 64, p, 0, None) == k3.K3MOE_E_ALIGN
    assert lib.k3moe_dequant_mxfp4(None, p, 4, 64, p, 0, None) == k3.K3MOE_E_NULL
    mx = lib.k3moe_forward_chunk_mx
    assert mx(ctypes.byref(s), p, 32, p, p, 16, 3, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert mx(ctypes.byref(s), p, 32, p, p, 16, 0, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert mx(ctypes.byref(_struct(D=3584 + 32)), p, 32, p, p, 16, 1, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert mx(ctypes.byref(_struct(F=3072 + 64)), p, 32, p, p, 16, 1, p, None, p, ws, None) == k3.K3MOE_E_DIM
    assert mx(ctypes.byref(s), p, 32, p, p, 16, 1, p, None, p, 100, None) == k3.K3MOE_E_WORKSPACE
    assert mx(ctypes.byref(s), None, 32, p, p, 16, 1, p, None, p, ws, None) == k3.K3MOE_E_NULL
    q = lib.k3moe_mx_quant
    assert q(None, 0, 64, 1, p, p, None) == k3.K3MOE_E_NULL
    assert q(p, 0, 48, 1, p, p, None) == k3.K3MOE_E_DIM
    assert q(p, 0, 0, 1, p, p, None) == k3.K3MOE_E_DIM
    assert q(p, 0, 64, 3, p, p, None) == k3.K3MOE_E_DIM
    assert q(p, 5, 64, 1, p, p, None) == k3.K3MOE_E_DIM
    assert q(ctypes.c_void_p(260), 0, 64, 1, p, p, None) == k3.K3MOE_E_ALIGN


def test_latent_validation():
    """k3moe_latent_forward / k3moe_latent_workspace_size reject bad arguments on the host."""
    lib = k3.load()
    s = _struct()
    p = 256
    L = k3.LatentStruct(7168, 6144, 1e-6, p, p, p, p, p, p)
    need = lib.k3moe_latent_workspace_size(ctypes.byref(L), 32, 16, ctypes.byref(s))
    assert need >= 32 * 6144 * 4 * 2 + 32 * 3584 * 4
    assert lib.k3moe_latent_workspace_size(ctypes.byref(L), 32, 65, ctypes.byref(s)) == 0
    for bad in (k3.LatentStruct(7000, 6144, 1e-6, p, p, p, p, p, p), k3.LatentStruct(7168, 6144, -1.0, p, p, p, p, p, p),
                k3.LatentStruct(7168, 6144, float("nan"), p, p, p, p, p, p)):
        assert lib.k3moe_latent_workspace_size(ctypes.byref(bad), 32, 16, ctypes.byref(s)) == 0
        assert lib.k3moe_latent_forward(ctypes.byref(bad), ctypes.byref(s), ctypes.c_void_p(p), 32, ctypes.c_void_p(p),
                                        ctypes.c_void_p(p), 16, ctypes.c_void_p(p), ctypes.c_void_p(p), need,
                                        None) == k3.K3MOE_E_DIM
    vp = ctypes.c_void_p(p)
    f = lib.k3moe_latent_forward
    assert f(None, ctypes.byref(s), vp, 32, vp, vp, 16, vp, vp, need, None) == k3.K3MOE_E_NULL
    assert f(ctypes.byref(L), ctypes.byref(s), None, 32, vp, vp, 16, vp, vp, need, None) == k3.K3MOE_E_NULL
    nul = k3.LatentStruct(7168, 6144, 1e-6, p, p, None, p, p, p)
    assert f(ctypes.byref(nul), ctypes.byref(s), vp, 32, vp, vp, 16, vp, vp, need, None) == k3.K3MOE_E_NULL
    mis = k3.LatentStruct(7168, 6144, 1e-6, p, p + 2, p, p, p, p)
    assert f(ctypes.byref(mis), ctypes.byref(s), vp, 32, vp, vp, 16, vp, vp, need, None) == k3.K3MOE_E_ALIGN
    assert f(ctypes.byref(L), ctypes.byref(s), vp, 0, vp, vp, 16, vp, vp, need, None) == k3.K3MOE_E_DIM
    assert f(ctypes.byref(L), ctypes.byref(s), vp, 32, vp, vp, 16, vp, vp, need - 1, None) == k3.K3MOE_E_WORKSPACE
    # T*max(d_hidden, d_shared) beyond 2^31 elements (32-bit row offsets of the dense products)
    assert f(ctypes.byref(L), ctypes.byref(_struct()), vp, (1 << 31) // 7168 + 1, vp, vp, 1, vp, vp, 1 << 62,
             None) == k3.K3MOE_E_DIM


def test_chunk_row_offsets_bound():
    """T*K*max(D, F) above 2^31 elements is a size error on every chunk entry point (the
    GEMM kernels address activation rows with 32-bit byte offsets); just under it the
    dimensions pass and the small workspace is what is refused."""
    lib = k3.load()
    s = _struct()
    p = 256
    limit = (1 << 31) // (16 * 3584)  # K = 16, max(D, F) = 3584
    over, under = limit + 1, limit
    ck, cb, mx = lib.k3moe_forward_chunk, lib.k3moe_forward_chunk_bf16, lib.k3moe_forward_chunk_mx
    for fn in (ck, cb):
        assert fn(ctypes.byref(s), p, over, p, p, 16, p, None, p, 1 << 62, None) == k3.K3MOE_E_DIM
        assert fn(ctypes.byref(s), p, under, p, p, 16, p, None, p, 100, None) == k3.K3MOE_E_WORKSPACE
    assert mx(ctypes.byref(s), p, over, p, p, 16, 1, p, None, p, 1 << 62, None) == k3.K3MOE_E_DIM
    assert mx(ctypes.byref(s), p, under, p, p, 16, 1, p, None, p, 100, None) == k3.K3MOE_E_WORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        k3.route(torch.zeros(1, 8), torch.zeros(8), 2)
