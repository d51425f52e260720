"""ctypes binding of ``libk3moe.so`` (the C ABI in ``include/k3moe.h``).

Argument marshalling only: every step of the routed-expert block runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current stream.
If the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3moe.so")

K3MOE_OK = 0
K3MOE_E_NULL = -1
K3MOE_E_DIM = -2
K3MOE_E_ALIGN = -3
K3MOE_E_WORKSPACE = -4
K3MOE_E_DEVICE = -5
K3MOE_E_HIP = -6
K3MOE_E_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = (2 << 20) + (64 << 10)  # K3MOE_NOALLOC_SCRATCH_BYTES
K3MOE_MAX_K = 64
K3MOE_MAX_E = 4096
K3MOE_MAX_DIM = 8192
OP_DECODE, OP_CHUNK, OP_GROUP, OP_CHUNK_MX = 1, 2, 3, 4
OUT_F32, OUT_BF16 = 0, 1
IN_F32, IN_BF16 = 0, 1

PRUNED = -1  # K3MOE_PRUNED: a routing slot dropped by top-p

ENTRY_POINTS = ("k3moe_route", "k3moe_route_topp", "k3moe_group", "k3moe_forward_decode", "k3moe_decode_gateup",
                "k3moe_decode_down", "k3moe_forward_chunk", "k3moe_forward_chunk_bf16", "k3moe_workspace_size", "k3moe_dequant_mxfp4",
                "k3moe_status_string", "k3moe_slot_layout", "k3moe_pool_create", "k3moe_pool_destroy",
                "k3moe_pool_plan", "k3moe_pool_weights", "k3moe_pool_stats", "k3moe_forward_decode_pooled",
                "k3moe_forward_chunk_mx", "k3moe_mx_quant", "k3moe_latent_forward", "k3moe_latent_workspace_size",
                "k3moe_forward_decode_timed", "k3moe_probe_stream_read", "k3moe_probe_mfma",
                "k3moe_forward_decode_noalloc")


class K3moeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} (status {code})")
        self.code = code


class LatentStruct(ctypes.Structure):
    _fields_ = ([("d_hidden", ctypes.c_int32), ("d_shared", ctypes.c_int32), ("eps", ctypes.c_float)] +
                [(n, ctypes.c_void_p) for n in ("w_down", "w_up", "norm", "shared_gate", "shared_up", "shared_down")])


class WeightsStruct(ctypes.Structure):
    _fields_ = ([("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32)] +
                [(n, ctypes.c_void_p) for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")] +
                [(n + "_stride", ctypes.c_int64)
                 for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")])


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    wp = ctypes.POINTER(WeightsStruct)
    lib.k3moe_route.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.k3moe_group.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.k3moe_forward_decode.argtypes = [wp, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.k3moe_forward_chunk.argtypes = [wp, vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.k3moe_forward_chunk_bf16.argtypes = [wp, vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.k3moe_decode_gateup.argtypes = [wp, vp, vp, i32, vp, vp]
    lib.k3moe_forward_decode_timed.argtypes = [wp, vp, vp, vp, i32, vp, vp, sz, vp, vp, vp]
    lib.k3moe_decode_down.argtypes = [wp, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.k3moe_forward_decode_noalloc.argtypes = [wp, vp, vp, vp, i32, vp, vp]
    lib.k3moe_workspace_size.argtypes = [i32, i32, i32, wp]
    lib.k3moe_workspace_size.restype = sz
    lib.k3moe_dequant_mxfp4.argtypes = [vp, vp, i32, i32, vp, i32, vp]
    lib.k3moe_status_string.argtypes = [ctypes.c_int]
    lib.k3moe_status_string.restype = ctypes.c_char_p
    i64 = ctypes.c_int64
    lib.k3moe_route_topp.argtypes = [vp, vp, i32, i32, i32, ctypes.c_double, vp, vp, vp, vp]
    lib.k3moe_slot_layout.argtypes = [i32, i32, vp]
    lib.k3moe_pool_create.argtypes = [i32, i32, i32, vp]
    lib.k3moe_pool_create.restype = vp
    lib.k3moe_pool_destroy.argtypes = [vp]
    lib.k3moe_pool_destroy.restype = None
    lib.k3moe_pool_plan.argtypes = [vp, i32, vp, i32, vp, vp]
    lib.k3moe_pool_weights.argtypes = [vp, wp]
    lib.k3moe_pool_stats.argtypes = [vp, vp]
    lib.k3moe_forward_decode_pooled.argtypes = [vp, i32, vp, i64, i64, vp, vp, vp, i32, vp, vp, sz, vp, vp]
    lib.k3moe_forward_chunk_mx.argtypes = [wp, vp, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.k3moe_mx_quant.argtypes = [vp, i32, i64, i32, vp, vp, vp]
    lp = ctypes.POINTER(LatentStruct)
    lib.k3moe_latent_forward.argtypes = [lp, wp, vp, i32, vp, vp, i32, vp, vp, sz, vp]
    lib.k3moe_latent_workspace_size.argtypes = [lp, i32, i32, wp]
    lib.k3moe_latent_workspace_size.restype = sz
    lib.k3moe_probe_stream_read.argtypes = [vp, sz, i32, i32, i32, vp, vp]
    lib.k3moe_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
    for name in ENTRY_POINTS:
        if name not in ("k3moe_workspace_size", "k3moe_status_string", "k3moe_pool_create", "k3moe_pool_destroy",
                        "k3moe_latent_workspace_size"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().k3moe_status_string(int(code)).decode()


def _check(fn: str, rc: int):
    if rc != K3MOE_OK:
        raise K3moeError(fn, rc)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


class ExpertWeights:
    """One layer's routed experts: six uint8 device tensors
    ``gate_q [E,F,D/2]``, ``gate_s [E,F,D/32]``, ``up_q``, ``up_s`` (same shapes),
    ``down_q [E,D,F/2]``, ``down_s [E,D,F/32]``."""

    NAMES = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")

    def __init__(self, gate_q, gate_s, up_q, up_s, down_q, down_s):
        E, F, half = gate_q.shape
        D = 2 * half
        shapes = {"gate_q": (E, F, D // 2), "gate_s": (E, F, D // 32), "up_q": (E, F, D // 2),
                  "up_s": (E, F, D // 32), "down_q": (E, D, F // 2), "down_s": (E, D, F // 32)}
        self.tensors = {}
        for n, t in zip(self.NAMES, (gate_q, gate_s, up_q, up_s, down_q, down_s)):
            self.tensors[n] = _dev(t, torch.uint8, n, shapes[n])
        self.E, self.D, self.F = E, D, F
        s = WeightsStruct()
        s.n_experts, s.d_model, s.d_ff = E, D, F
        for n in self.NAMES:
            t = self.tensors[n]
            setattr(s, n, t.data_ptr())
            setattr(s, n + "_stride", t.stride(0) * t.element_size())
        self.struct = s

    @classmethod
    def from_dict(cls, d: Dict[str, torch.Tensor]) -> "ExpertWeights":
        return cls(*(d[n] for n in cls.NAMES))

    @classmethod
    def from_struct(cls, struct: "WeightsStruct", keepalive=None) -> "ExpertWeights":
        """Weights described by a filled k3moe_weights_t (e.g. a residency pool's
        slots); ``keepalive`` holds the memory it points into."""
        self = cls.__new__(cls)
        self.tensors = {}
        self.E, self.D, self.F = struct.n_experts, struct.d_model, struct.d_ff
        self.struct = struct
        self.keepalive = keepalive
        return self

    def ref(self):
        return ctypes.byref(self.struct)


def workspace_size(op: int, T: int, K: int, W: ExpertWeights) -> int:
    return int(load().k3moe_workspace_size(int(op), int(T), int(K), W.ref()))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return _dev(ws, torch.uint8, "workspace")


def route(logits: torch.Tensor, bias: torch.Tensor, K: int, idx: Optional[torch.Tensor] = None,
          w: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sigmoid + bias top-K router: ``logits [T,E]`` -> ``(idx [T,K] int32, w [T,K] f32)``."""
    T, E = logits.shape
    _dev(logits, torch.float32, "logits")
    _dev(bias, torch.float32, "bias", (E,))
    idx = torch.empty((T, K), dtype=torch.int32, device=logits.device) if idx is None else idx
    w = torch.empty((T, K), dtype=torch.float32, device=logits.device) if w is None else w
    _dev(idx, torch.int32, "idx", (T, K))
    _dev(w, torch.float32, "w", (T, K))
    _check("k3moe_route", load().k3moe_route(_ptr(logits), _ptr(bias), T, E, K, _ptr(idx), _ptr(w),
                                              _stream(stream)))
    return idx, w


def route_topp(logits: torch.Tensor, bias: torch.Tensor, K: int, top_p: float, idx: Optional[torch.Tensor] = None,
               w: Optional[torch.Tensor] = None, n_kept: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Router plus top-p pruning: ``(idx [T,K], w [T,K], n_kept [T])``; pruned slots
    (after the kept ones) hold ``PRUNED`` and weight 0."""
    T, E = logits.shape
    _dev(logits, torch.float32, "logits")
    _dev(bias, torch.float32, "bias", (E,))
    dev = logits.device
    idx = torch.empty((T, K), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, K), dtype=torch.float32, device=dev) if w is None else w
    n_kept = torch.empty(T, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    _dev(idx, torch.int32, "idx", (T, K))
    _dev(w, torch.float32, "w", (T, K))
    _dev(n_kept, torch.int32, "n_kept", (T,))
    _check("k3moe_route_topp", load().k3moe_route_topp(_ptr(logits), _ptr(bias), T, E, K, ctypes.c_double(top_p),
                                                        _ptr(idx), _ptr(w), _ptr(n_kept), _stream(stream)))
    return idx, w, n_kept


def group(idx: torch.Tensor, E: int, ws: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """Counting-sort grouping of a chunk's pairs by expert (device tensors)."""
    T, K = idx.shape
    _dev(idx, torch.int32, "idx")
    dev = idx.device
    out = {"counts": torch.empty(E, dtype=torch.int32, device=dev),
           "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "perm": torch.empty(T * K, dtype=torch.int32, device=dev),
           "uniq": torch.empty(E, dtype=torch.int32, device=dev),
           "n_unique": torch.empty(1, dtype=torch.int32, device=dev)}
    s = WeightsStruct()
    s.n_experts, s.d_model, s.d_ff = E, 32, 32
    nbytes = int(load().k3moe_workspace_size(OP_GROUP, T, K, ctypes.byref(s)))
    ws = _workspace(nbytes, dev, ws)
    _check("k3moe_group", load().k3moe_group(_ptr(idx), T, K, E, _ptr(out["counts"]), _ptr(out["offsets"]),
                                              _ptr(out["perm"]), _ptr(out["uniq"]), _ptr(out["n_unique"]),
                                              _ptr(ws), ws.numel(), _stream(stream)))
    return out


def forward_decode(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                   y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """One token: ``x [D]`` with its ``idx [K]`` / ``w [K]`` -> ``y [D]`` (fp32 path)."""
    x = _dev(x.reshape(-1) if x.dim() == 2 and x.shape[0] == 1 else x, torch.float32, "x", (W.D,))
    idx = idx.reshape(-1)
    w = w.reshape(-1)
    K = idx.numel()
    _dev(idx, torch.int32, "idx", (K,))
    _dev(w, torch.float32, "w", (K,))
    y = torch.empty(W.D, dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (W.D,))
    ws = _workspace(workspace_size(OP_DECODE, 1, K, W), x.device, ws)
    _check("k3moe_forward_decode",
           load().k3moe_forward_decode(W.ref(), _ptr(x), _ptr(idx), _ptr(w), K, _ptr(y), _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return y


def forward_decode_noalloc(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                           y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """forward_decode on the library's fixed per-device scratch (no workspace
    argument; the C entry point allocates nothing -- pass ``y`` to allocate nothing
    here either).  Calls that overlap on one device race."""
    x = _dev(x.reshape(-1) if x.dim() == 2 and x.shape[0] == 1 else x, torch.float32, "x", (W.D,))
    idx = idx.reshape(-1)
    w = w.reshape(-1)
    K = idx.numel()
    _dev(idx, torch.int32, "idx", (K,))
    _dev(w, torch.float32, "w", (K,))
    y = torch.empty(W.D, dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (W.D,))
    _check("k3moe_forward_decode_noalloc",
           load().k3moe_forward_decode_noalloc(W.ref(), _ptr(x), _ptr(idx), _ptr(w), K, _ptr(y), _stream(stream)))
    return y


def forward_decode_timed(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor, ev_start: int,
                         ev_stop: int, y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """forward_decode with the gate/up kernel's own start and end recorded in two
    caller-owned hipEvent_t handles (raw pointers as ints)."""
    x = _dev(x.reshape(-1) if x.dim() == 2 and x.shape[0] == 1 else x, torch.float32, "x", (W.D,))
    idx = idx.reshape(-1)
    w = w.reshape(-1)
    K = idx.numel()
    _dev(idx, torch.int32, "idx", (K,))
    _dev(w, torch.float32, "w", (K,))
    y = torch.empty(W.D, dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (W.D,))
    ws = _workspace(workspace_size(OP_DECODE, 1, K, W), x.device, ws)
    _check("k3moe_forward_decode_timed",
           load().k3moe_forward_decode_timed(W.ref(), _ptr(x), _ptr(idx), _ptr(w), K, _ptr(y), _ptr(ws), ws.numel(),
                                             ctypes.c_void_p(ev_start), ctypes.c_void_p(ev_stop), _stream(stream)))
    return y


def decode_gateup(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, h: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Decode stage 1: ``h [K, F]`` = SiTU-GLU of the K experts' gate/up rows on ``x [D]``."""
    _dev(x, torch.float32, "x", (W.D,))
    idx = idx.reshape(-1)
    K = idx.numel()
    _dev(idx, torch.int32, "idx", (K,))
    h = torch.empty((K, W.F), dtype=torch.float32, device=x.device) if h is None else h
    _dev(h, torch.float32, "h", (K, W.F))
    _check("k3moe_decode_gateup", load().k3moe_decode_gateup(W.ref(), _ptr(x), _ptr(idx), K, _ptr(h), _stream(stream)))
    return h


def decode_down(W: ExpertWeights, h: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode stage 2: ``y [D]`` = sum_k w_k W_down[e_k] h[k] (slot order)."""
    idx = idx.reshape(-1)
    w = w.reshape(-1)
    K = idx.numel()
    _dev(h, torch.float32, "h", (K, W.F))
    _dev(idx, torch.int32, "idx", (K,))
    _dev(w, torch.float32, "w", (K,))
    y = torch.empty(W.D, dtype=torch.float32, device=h.device) if y is None else y
    _dev(y, torch.float32, "y", (W.D,))
    ws = _workspace(workspace_size(OP_DECODE, 1, K, W), h.device, ws)
    _check("k3moe_decode_down", load().k3moe_decode_down(W.ref(), _ptr(h), _ptr(idx), _ptr(w), K, _ptr(y), _ptr(ws),
                                                          ws.numel(), _stream(stream)))
    return y


def forward_chunk(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                  y: Optional[torch.Tensor] = None, n_unique: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A chunk: ``x [T,D]``, ``idx/w [T,K]`` -> fp32 ``y [T,D]`` (grouped MFMA path).  An
    fp32 ``x`` goes to ``k3moe_forward_chunk`` (fp16 items, or bf16 high part + MXFP4 low
    part), a bf16 ``x`` to ``k3moe_forward_chunk_bf16``."""
    T = x.shape[0]
    fn = "k3moe_forward_chunk_bf16" if x.dtype == torch.bfloat16 else "k3moe_forward_chunk"
    _dev(x, torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32, "x", (T, W.D))
    K = idx.shape[1]
    _dev(idx, torch.int32, "idx", (T, K))
    _dev(w, torch.float32, "w", (T, K))
    y = torch.empty((T, W.D), dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (T, W.D))
    if n_unique is not None:
        _dev(n_unique, torch.int32, "n_unique", (1,))
    ws = _workspace(workspace_size(OP_CHUNK, T, K, W), x.device, ws)
    _check(fn, getattr(load(), fn)(W.ref(), _ptr(x), T, _ptr(idx), _ptr(w), K, _ptr(y), _ptr(n_unique),
                                   _ptr(ws), ws.numel(), _stream(stream)))
    return y


def forward_chunk_mx(W: ExpertWeights, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor, parts: int = 1,
                     y: Optional[torch.Tensor] = None, n_unique: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A chunk with MXFP8 activations in ``parts`` parts: fp32 ``x [T,D]``,
    ``idx/w [T,K]`` -> fp32 ``y [T,D]`` (scaled FP8 x FP4 MFMA path)."""
    T = x.shape[0]
    _dev(x, torch.float32, "x", (T, W.D))
    K = idx.shape[1]
    _dev(idx, torch.int32, "idx", (T, K))
    _dev(w, torch.float32, "w", (T, K))
    y = torch.empty((T, W.D), dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (T, W.D))
    if n_unique is not None:
        _dev(n_unique, torch.int32, "n_unique", (1,))
    ws = _workspace(workspace_size(OP_CHUNK_MX, T, K, W), x.device, ws)
    _check("k3moe_forward_chunk_mx",
           load().k3moe_forward_chunk_mx(W.ref(), _ptr(x), T, _ptr(idx), _ptr(w), K, int(parts), _ptr(y),
                                         _ptr(n_unique), _ptr(ws), ws.numel(), _stream(stream)))
    return y


class LatentWeights:
    """The dense bf16 weights of a LatentMoE block (device tensors, kept alive here):
    ``w_down [Dl,Dh]``, ``w_up [Dh,Dl]``, ``norm [Dl]``, ``shared_gate/shared_up [Fs,Dh]``,
    ``shared_down [Dh,Fs]``, and the RMSNorm ``eps``."""

    NAMES = ("w_down", "w_up", "norm", "shared_gate", "shared_up", "shared_down")

    def __init__(self, tensors: Dict[str, torch.Tensor], eps: float):
        self.t = {n: tensors[n] for n in self.NAMES}
        for n, v in self.t.items():
            _dev(v, torch.bfloat16, n)
        self.Dl, self.Dh = self.t["w_down"].shape
        self.Fs = self.t["shared_gate"].shape[0]
        if (tuple(self.t["w_up"].shape) != (self.Dh, self.Dl) or tuple(self.t["norm"].shape) != (self.Dl,)
                or tuple(self.t["shared_up"].shape) != (self.Fs, self.Dh)
                or tuple(self.t["shared_down"].shape) != (self.Dh, self.Fs)):
            raise ValueError("dense weight shapes do not match")
        self.s = LatentStruct(self.Dh, self.Fs, float(eps), *[_ptr(self.t[n]) for n in self.NAMES])

    def ref(self):
        return ctypes.byref(self.s)


def latent_forward(L: LatentWeights, W: ExpertWeights, h: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                   out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The LatentMoE block: bf16 ``h [T,Dh]``, routing ``idx/w [T,K]`` -> fp32 ``out [T,Dh]``."""
    T = h.shape[0]
    _dev(h, torch.bfloat16, "h", (T, L.Dh))
    if W.D != L.Dl:
        raise ValueError("the routed experts' d_model must equal the latent width")
    K = idx.shape[1]
    _dev(idx, torch.int32, "idx", (T, K))
    _dev(w, torch.float32, "w", (T, K))
    out = torch.empty((T, L.Dh), dtype=torch.float32, device=h.device) if out is None else out
    _dev(out, torch.float32, "out", (T, L.Dh))
    need = load().k3moe_latent_workspace_size(L.ref(), T, K, W.ref())
    if need == 0:
        raise ValueError("invalid LatentMoE arguments")
    ws = _workspace(need, h.device, ws)
    _check("k3moe_latent_forward",
           load().k3moe_latent_forward(L.ref(), W.ref(), _ptr(h), T, _ptr(idx), _ptr(w), K, _ptr(out), _ptr(ws),
                                       ws.numel(), _stream(stream)))
    return out


def mx_quant(v: torch.Tensor, parts: int = 1, stream=None):
    """OCP MXFP8 of a device fp32 or bf16 tensor whose element count is a multiple
    of 32 (groups of 32 consecutive elements).  Returns ``(codes, scales)`` uint8 of
    shapes ``[parts, n]`` and ``[parts, n/32]``."""
    code = {torch.float32: IN_F32, torch.bfloat16: IN_BF16}.get(v.dtype)
    if code is None:
        raise TypeError("v must be float32 or bfloat16")
    _dev(v, v.dtype, "v")
    n = v.numel()
    codes = torch.empty((parts, n), dtype=torch.uint8, device=v.device)
    scales = torch.empty((parts, max(n // 32, 1)), dtype=torch.uint8, device=v.device)
    _check("k3moe_mx_quant",
           load().k3moe_mx_quant(_ptr(v), code, n, int(parts), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def dequant_mxfp4(q: torch.Tensor, s: torch.Tensor, out_dtype: torch.dtype = torch.float32,
                  stream=None) -> torch.Tensor:
    """Decode ``q [O, I/2]`` + ``s [O, I/32]`` to ``[O, I]`` fp32 or bf16."""
    O, half = q.shape
    I = 2 * half
    _dev(q, torch.uint8, "q")
    _dev(s, torch.uint8, "s", (O, I // 32))
    code = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    out = torch.empty((O, I), dtype=out_dtype, device=q.device)
    _check("k3moe_dequant_mxfp4",
           load().k3moe_dequant_mxfp4(_ptr(q), _ptr(s), O, I, _ptr(out), code, _stream(stream)))
    return out


# ---------------------------------------------------------------- expert residency
def slot_layout(D: int, F: int):
    """Byte offsets of the six tensors within an expert slot, and the slot size."""
    off = (ctypes.c_int64 * 7)()
    _check("k3moe_slot_layout", load().k3moe_slot_layout(int(D), int(F), off))
    return [int(v) for v in off]


class Pool:
    """An LRU pool of ``n_slots`` HBM expert slots over the uint8 device tensor
    ``slots`` (at least ``n_slots * slot_bytes`` bytes, 256-byte aligned)."""

    def __init__(self, n_slots: int, D: int, F: int, slots: torch.Tensor):
        _dev(slots, torch.uint8, "slots")
        self.layout = slot_layout(D, F)
        if slots.numel() < n_slots * self.layout[6]:
            raise ValueError("slots tensor too small")
        self.slots = slots
        self.n_slots, self.D, self.F = n_slots, D, F
        self.handle = load().k3moe_pool_create(int(n_slots), int(D), int(F), _ptr(slots))
        if not self.handle:
            raise ValueError("k3moe_pool_create rejected its arguments")

    def plan(self, layer: int, experts):
        import numpy as np
        e = np.ascontiguousarray(experts, dtype=np.int32)
        slots = np.empty_like(e)
        missed = np.empty_like(e)
        _check("k3moe_pool_plan", load().k3moe_pool_plan(self.handle, int(layer), e.ctypes.data, e.size,
                                                          slots.ctypes.data, missed.ctypes.data))
        return slots, missed

    def weights(self) -> ExpertWeights:
        s = WeightsStruct()
        _check("k3moe_pool_weights", load().k3moe_pool_weights(self.handle, ctypes.byref(s)))
        return ExpertWeights.from_struct(s, keepalive=self.slots)

    def stats(self):
        out = (ctypes.c_int64 * 3)()
        _check("k3moe_pool_stats", load().k3moe_pool_stats(self.handle, out))
        return {"hits": int(out[0]), "misses": int(out[1]), "bytes": int(out[2])}

    def close(self):
        if getattr(self, "handle", None):
            load().k3moe_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward_decode_pooled(pool: Pool, layer: int, host: torch.Tensor, layer_stride: int, expert_stride: int,
                          x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor, y: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None, stream=None, copy_stream=None) -> torch.Tensor:
    """``forward_decode`` for one token whose layer-``layer`` experts live in the
    pinned host tensor ``host`` (slot layout, at layer*layer_stride +
    expert*expert_stride); missing experts are copied into the pool on
    ``copy_stream`` while the resident ones compute."""
    if not isinstance(host, torch.Tensor) or host.is_cuda or not host.is_pinned():
        raise TypeError("host must be a pinned CPU tensor")
    x = _dev(x, torch.float32, "x", (pool.D,))
    idx = idx.reshape(-1)
    w = w.reshape(-1)
    K = idx.numel()
    _dev(idx, torch.int32, "idx", (K,))
    _dev(w, torch.float32, "w", (K,))
    y = torch.empty(pool.D, dtype=torch.float32, device=x.device) if y is None else y
    _dev(y, torch.float32, "y", (pool.D,))
    W = pool.weights()
    ws = _workspace(workspace_size(OP_DECODE, 1, K, W) + 768, x.device, ws)
    cs = _stream(copy_stream if copy_stream is not None else stream)
    _check("k3moe_forward_decode_pooled",
           load().k3moe_forward_decode_pooled(pool.handle, int(layer), ctypes.c_void_p(host.data_ptr()),
                                              int(layer_stride), int(expert_stride), _ptr(x), _ptr(idx), _ptr(w),
                                              K, _ptr(y), _ptr(ws), ws.numel(), _stream(stream), cs))
    return y


def probe_stream_read(buf: torch.Tensor, unroll: int = 8, nontemporal: bool = False, blocks: int = 2048,
                      sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Launch the streaming-read probe over the bytes of ``buf`` (measurement only)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA tensor")
    sink = torch.empty(blocks, dtype=torch.int32, device=buf.device) if sink is None else sink
    _check("k3moe_probe_stream_read",
           load().k3moe_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(unroll),
                                          int(bool(nontemporal)), int(blocks), _ptr(sink), _stream(stream)))
    return sink


def probe_mfma(kind: int, iters: int, blocks: int, out: Optional[torch.Tensor] = None, stream=None,
               device="cuda") -> torch.Tensor:
    """Launch the MFMA issue-rate probe (measurement only)."""
    out = torch.empty(4 * blocks, dtype=torch.float32, device=device) if out is None else out
    _check("k3moe_probe_mfma", load().k3moe_probe_mfma(int(kind), int(iters), int(blocks), _ptr(out),
                                                       _stream(stream)))
    return out
