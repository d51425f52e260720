"""CPU oracle for the MXFP4 routed-expert block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never imports it, and the two share no code.

The arithmetic lives in ``k3moe_oracle.c`` (plain C, fp64 accumulation, built at
-O2 without fast-math); this module builds it with gcc and marshals numpy arrays.
Each C function cites the page passage it follows.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, invariants and hand-built fixtures.  The
end-to-end block output has no worked example on the pages, so beyond the
composition of those pins it is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_k3moe_oracle.so")

_F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle source ``src`` with gcc into ``out`` (default ``oracle/_k3moe_oracle.so``)."""
    global _default
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == _LIB_PATH:
        _default = None
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.k3o_decode.restype = ctypes.c_float
    lib.k3o_decode.argtypes = [ctypes.c_uint, ctypes.c_uint]
    lib.k3o_decode_table.restype = None
    lib.k3o_decode_table.argtypes = [_F32P]
    lib.k3o_dequant.restype = None
    lib.k3o_dequant.argtypes = [_U8P, _U8P, ctypes.c_int64, ctypes.c_int64, _F32P]
    lib.k3o_route.restype = None
    lib.k3o_route.argtypes = [_F32P, _F32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                              _I32P, _F32P, _F64P]
    lib.k3o_route_topp.restype = None
    lib.k3o_route_topp.argtypes = [_F32P, _F32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                   _I32P, _F32P, _I32P, _F64P]
    lib.k3o_situ.restype = ctypes.c_double
    lib.k3o_situ.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.k3o_situ_beta.restype = ctypes.c_double
    lib.k3o_situ_beta.argtypes = [ctypes.c_double] * 4
    lib.k3o_expert.restype = None
    lib.k3o_expert.argtypes = [_F32P, _F32P, _F32P, ctypes.c_int32, ctypes.c_int32, _F32P,
                               _F64P, _F64P, _F64P, _F64P]
    lib.k3o_forward.restype = ctypes.c_int
    lib.k3o_forward.argtypes = ([ctypes.c_int32] * 3 + [_U8P] * 6 +
                                [_F32P, ctypes.c_int32, _I32P, _F32P, ctypes.c_int32, _F32P,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32])
    lib.k3o_forward_mx.restype = ctypes.c_int
    lib.k3o_forward_mx.argtypes = lib.k3o_forward.argtypes + [ctypes.c_int32]
    lib.k3o_mx_quant_parts.restype = None
    lib.k3o_mx_quant_parts.argtypes = [_F32P, ctypes.c_int64, ctypes.c_int32, _U8P, _U8P]
    lib.k3o_mx_quant.restype = None
    lib.k3o_mx_quant.argtypes = [_F32P, ctypes.c_int64, _U8P, _U8P]
    lib.k3o_e4m3_decode.restype = ctypes.c_double
    lib.k3o_e4m3_decode.argtypes = [ctypes.c_uint]
    lib.k3o_rmsnorm.restype = ctypes.c_double
    lib.k3o_rmsnorm.argtypes = [_F64P, ctypes.c_int32, _F32P, ctypes.c_double, _F64P]
    lib.k3o_latent_forward.restype = ctypes.c_int
    lib.k3o_latent_forward.argtypes = ([ctypes.c_int32] * 3 + [_F32P, _F32P, _F32P, ctypes.c_double, _F32P, _F32P, _F32P]
                                       + [ctypes.c_int32] * 2 + [_U8P] * 6
                                       + [_F32P, ctypes.c_int32, _I32P, _F32P, ctypes.c_int32, _F32P,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32])
    lib.k3o_set_progress.restype = None
    lib.k3o_set_progress.argtypes = [ctypes.c_int32]
    lib.k3o_group.restype = ctypes.c_int
    lib.k3o_group.argtypes = [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P,
                              _I32P, _I32P, ctypes.POINTER(ctypes.c_int32)]
    return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """The oracle's functions bound to one compiled library (the default build, or a
    copy built from another source file, as the pin self-tests do)."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self.lib = _bind(lib_path)

    # ------------------------------------------------------------------------- decode
    def decode(self, code: int, scale: int) -> np.float32:
        return np.float32(self.lib.k3o_decode(int(code), int(scale)))

    def decode_table(self) -> np.ndarray:
        """``[16, 256]`` fp32: entry ``[c, s]`` is the weight of code c at scale byte s."""
        out = np.empty(16 * 256, dtype=np.float32)
        self.lib.k3o_decode_table(out)
        return out.reshape(16, 256)

    def dequant(self, q: np.ndarray, s: np.ndarray) -> np.ndarray:
        """MXFP4 ``q [O, I/2]`` + ``s [O, I/32]`` -> fp32 ``[O, I]``."""
        q = _c(q, np.uint8)
        s = _c(s, np.uint8)
        O, half = q.shape
        I = 2 * half
        if s.shape != (O, I // 32) or I % 32:
            raise ValueError("bad MXFP4 shapes")
        out = np.empty((O, I), dtype=np.float32)
        self.lib.k3o_dequant(q, s, O, I, out)
        return out

    # -------------------------------------------------------------------------- route
    def route(self, logits: np.ndarray, bias: np.ndarray, K: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """``(idx [T,K] int32, w [T,K] f32, gap [T] f64)`` for logits ``[T,E]``."""
        logits = _c(logits, np.float32)
        if logits.ndim == 1:
            logits = logits[None]
        T, E = logits.shape
        bias = _c(bias, np.float32)
        if bias.shape != (E,) or not 1 <= K <= E:
            raise ValueError("bad route arguments")
        idx = np.empty((T, K), dtype=np.int32)
        w = np.empty((T, K), dtype=np.float32)
        gap = np.empty(T, dtype=np.float64)
        self.lib.k3o_route(logits, bias, T, E, K, idx, w, gap)
        return idx, w, gap

    def route_topp(self, logits: np.ndarray, bias: np.ndarray, K: int,
                   p: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
        """Router plus top-p pruning: ``(idx, w, n_kept [T] int32, gap)``; pruned
        slots (after the kept ones) hold id -1 and weight 0."""
        logits = _c(logits, np.float32)
        if logits.ndim == 1:
            logits = logits[None]
        T, E = logits.shape
        bias = _c(bias, np.float32)
        if bias.shape != (E,) or not 1 <= K <= E:
            raise ValueError("bad route arguments")
        idx = np.empty((T, K), dtype=np.int32)
        w = np.empty((T, K), dtype=np.float32)
        n_kept = np.empty(T, dtype=np.int32)
        gap = np.empty(T, dtype=np.float64)
        self.lib.k3o_route_topp(logits, bias, T, E, K, float(p), idx, w, n_kept, gap)
        return idx, w, n_kept, gap

    # --------------------------------------------------------------------- activation
    def situ(self, g: float, u: float) -> float:
        return self.lib.k3o_situ(float(g), float(u))

    def situ_beta(self, g: float, u: float, bg: float, bu: float) -> float:
        return self.lib.k3o_situ_beta(float(g), float(u), float(bg), float(bu))

    # ------------------------------------------------------------------------- expert
    def expert(self, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray) -> Dict[str, np.ndarray]:
        """One expert on one token from decoded fp32 weights; returns g, u, h, y (float64)."""
        Wg, Wu, Wd, x = (_c(a, np.float32) for a in (Wg, Wu, Wd, x))
        F, D = Wg.shape
        if Wu.shape != (F, D) or Wd.shape != (D, F) or x.shape != (D,):
            raise ValueError("bad expert shapes")
        g, u, h = (np.empty(F) for _ in range(3))
        y = np.empty(D)
        self.lib.k3o_expert(Wg, Wu, Wd, D, F, x, g, u, h, y)
        return {"g": g, "u": u, "h": h, "y": y}

    # ------------------------------------------------------------------------ forward
    def forward(self, weights: Dict[str, np.ndarray], x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                nthreads: Optional[int] = None, want_pairs: bool = False, mx: int = 0, progress: int = 0):
        """Routed-expert block on host weights ``{name: [E, rows, cols]}``.

        Returns ``y [T, D] f32``; with ``want_pairs`` also ``(ytk [T,K,D], hk [T,K,F])``
        in float64.  ``mx=1`` or ``mx=2`` runs the MXFP8-activation variant in that many
        parts (``k3o_forward_mx``: x and h quantized per 32 to E4M3 with an E8M0 scale;
        the weights keep the closed form for every scale byte).  ``progress=n`` reports
        every n-th finished expert on stderr.
        """
        names = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
        arrs = [_c(weights[n], np.uint8) for n in names]
        E, F, half = arrs[0].shape
        D = 2 * half
        x = _c(x, np.float32)
        if x.ndim == 1:
            x = x[None]
        idx = _c(idx, np.int32)
        if idx.ndim == 1:
            idx = idx[None]
        w = _c(w, np.float32).reshape(idx.shape)
        T, K = idx.shape
        if x.shape != (T, D):
            raise ValueError("x must be [T, D]")
        y = np.empty((T, D), dtype=np.float32)
        ytk = np.empty((T, K, D)) if want_pairs else None
        hk = np.empty((T, K, F)) if want_pairs else None
        args = [E, D, F, *arrs, x, T, idx, w, K, y, ytk.ctypes.data if want_pairs else None,
                hk.ctypes.data if want_pairs else None, int(nthreads or default_threads())]
        self.lib.k3o_set_progress(int(progress))
        try:
            rc = self.lib.k3o_forward_mx(*args, int(mx)) if mx else self.lib.k3o_forward(*args)
        finally:
            self.lib.k3o_set_progress(0)
        if rc != 0:
            raise ValueError("oracle forward failed (expert index out of range or out of memory)")
        return (y, ytk, hk) if want_pairs else y

    # ------------------------------------------------------------ MXFP8 activations
    def mx_quant(self, v: np.ndarray, parts: int = 1):
        """OCP MXFP8 (E4M3, E8M0 scale per 32) of a float32 array whose last dimension
        is a multiple of 32, in ``parts`` parts (2: the second part quantizes the
        residual).  Returns ``(codes u8, scales u8)``; with one part of shapes
        ``v.shape`` and ``v.shape[:-1] + (n/32,)``, with two parts with a leading 2."""
        v = _c(v, np.float32)
        if v.shape[-1] % 32:
            raise ValueError("last dimension must be a multiple of 32")
        if parts not in (1, 2):
            raise ValueError("parts must be 1 or 2")
        codes = np.empty((parts,) + v.shape, np.uint8)
        scales = np.empty((parts,) + v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
        self.lib.k3o_mx_quant_parts(v, v.size, parts, codes, scales)
        return (codes[0], scales[0]) if parts == 1 else (codes, scales)

    def e4m3(self, code: int) -> float:
        return float(self.lib.k3o_e4m3_decode(int(code)))

    # ------------------------------------------------------------- LatentMoE wrapper
    def rmsnorm(self, a: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
        a = _c(a, np.float64)
        r = np.empty_like(a)
        self.lib.k3o_rmsnorm(a, a.size, _c(g, np.float32), float(eps), r)
        return r

    def latent_forward(self, dense: Dict[str, np.ndarray], weights: Dict[str, np.ndarray], h: np.ndarray,
                       idx: np.ndarray, w: np.ndarray, nthreads: Optional[int] = None, want_parts: bool = False):
        """The LatentMoE block (k3o_latent_forward): ``dense`` holds ``w_dn [Dl,Dh]``,
        ``w_up [Dh,Dl]``, ``norm [Dl]``, ``eps``, ``sg/su [Fs,Dh]``, ``sd [Dh,Fs]`` (float
        values); ``weights`` the routed experts at width Dl.  Returns ``out [T,Dh]`` f32;
        with ``want_parts`` also ``(x_latent, aggregate)`` [T,Dl] in float64."""
        names = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
        arrs = [_c(weights[n], np.uint8) for n in names]
        E, F, half = arrs[0].shape
        Dl = 2 * half
        wdn, wup = _c(dense["w_dn"], np.float32), _c(dense["w_up"], np.float32)
        sg, su, sd = (_c(dense[k], np.float32) for k in ("sg", "su", "sd"))
        norm = _c(dense["norm"], np.float32)
        Dh, Fs = wdn.shape[1], sg.shape[0]
        if wdn.shape != (Dl, Dh) or wup.shape != (Dh, Dl) or norm.shape != (Dl,) or su.shape != (Fs, Dh) \
                or sd.shape != (Dh, Fs):
            raise ValueError("dense weight shapes do not match")
        h = _c(h, np.float32).reshape(-1, Dh)
        T = h.shape[0]
        idx = _c(idx, np.int32).reshape(T, -1)
        K = idx.shape[1]
        w = _c(w, np.float32).reshape(T, K)
        out = np.empty((T, Dh), np.float32)
        xl = np.empty((T, Dl)) if want_parts else None
        agg = np.empty((T, Dl)) if want_parts else None
        rc = self.lib.k3o_latent_forward(Dh, Dl, Fs, wdn, wup, norm, float(dense["eps"]), sg, su, sd, E, F, *arrs,
                                         h, T, idx, w, K, out, xl.ctypes.data if want_parts else None,
                                         agg.ctypes.data if want_parts else None, int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle latent forward failed")
        return (out, xl, agg) if want_parts else out

    # -------------------------------------------------------------------------- group
    def group(self, idx: np.ndarray, E: int) -> Dict[str, np.ndarray]:
        """Counting-sort grouping of a chunk's pairs by expert (see ``k3o_group``)."""
        idx = _c(idx, np.int32)
        T, K = idx.shape
        counts = np.empty(E, dtype=np.int32)
        offsets = np.empty(E + 1, dtype=np.int32)
        perm = np.full(T * K, -1, dtype=np.int32)
        uniq = np.full(E, -1, dtype=np.int32)
        nu = ctypes.c_int32(0)
        rc = self.lib.k3o_group(idx, T, K, E, counts, offsets, perm, uniq, ctypes.byref(nu))
        if rc != 0:
            raise ValueError("expert index out of range")
        perm = perm[:offsets[E]].copy()  # pruned slots are not placed
        return {"counts": counts, "offsets": offsets, "perm": perm,
                "uniq": uniq[:nu.value].copy(), "n_unique": int(nu.value)}


_default: Optional[Oracle] = None


def instance() -> Oracle:
    """The oracle built from ``k3moe_oracle.c`` (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def decode(code, scale):
    return instance().decode(code, scale)


def decode_table():
    return instance().decode_table()


def dequant(q, s):
    return instance().dequant(q, s)


def route(logits, bias, K):
    return instance().route(logits, bias, K)


def route_topp(logits, bias, K, p):
    return instance().route_topp(logits, bias, K, p)


def situ(g, u):
    return instance().situ(g, u)


def situ_beta(g, u, bg, bu):
    return instance().situ_beta(g, u, bg, bu)


def expert(Wg, Wu, Wd, x):
    return instance().expert(Wg, Wu, Wd, x)


def forward(weights, x, idx, w, nthreads=None, want_pairs=False, mx=0, progress=0):
    return instance().forward(weights, x, idx, w, nthreads=nthreads, want_pairs=want_pairs, mx=mx,
                              progress=progress)


def mx_quant(v, parts=1):
    return instance().mx_quant(v, parts=parts)


def latent_forward(dense, weights, h, idx, w, nthreads=None, want_parts=False):
    return instance().latent_forward(dense, weights, h, idx, w, nthreads=nthreads, want_parts=want_parts)


def group(idx, E):
    return instance().group(idx, E)
