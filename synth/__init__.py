"""Seeded synthetic inputs for the MXFP4 routed-expert block.

This module only draws numbers: it holds none of the block's arithmetic (no
decode, no routing, no matmul).  Both the CPU oracle and the HIP library are fed
from it, so the two sides always see byte-identical inputs.

Workloads (shapes from the Kimi K3 engine pages: 896 routed experts per layer,
top-16, a 3584-dim latent space; F = 3072 makes one expert 17 547 264 bytes of
MXFP4, i.e. 16 experts x 92 MoE layers = 25.8 GB streamed per token, the volume
colibri PR #676 reports in "It runs the full model"):

  tiny        1 token,   E=8,   K=2,  D=256,  F=128, decode path
  decode1     1 token,   E=896, K=16, D=3584, F=3072, decode path
  prefill32   32 tokens, same shape, AR(1) hidden states, logits = h.R, chunk path
  prefill256  256 tokens, same as prefill32, chunk path
  batch4096   4096 tokens, i.i.d. hidden states, logits = h.R, chunk path;
              eight "edge" experts carry scale bytes over the full 0..255 range

Hidden states are fp32 except for prefill256, whose workload names bf16
activations (those values are rounded to bf16 here, so both sides see them).

Edge experts (batch4096): in each scale tensor a quarter of the groups, drawn
independently, take a scale byte uniform over 0..255 (every byte value occurs a
few hundred times per tensor); the rest keep the workload's range.  In an edge
group whose scale byte exceeds 128 the codes are +-0 (nibbles 0 and 8 only), so
its weights are +-0 * 2^(s-127) = +-0 by the closed form, s = 255 included; edge
groups at or below 128 keep uniform codes (s = 0 gives fp32 subnormal weights).
All 16 codes and all 256 scale bytes appear, and a token routed to an edge
expert keeps a finite output that the parity tests measure.  edge_mode
"literal" instead draws every scale byte of an edge expert uniform over 0..255
(weights up to +-inf; most outputs NaN), for the non-finite mask check.

LatentMoE block workloads (the routed experts behind 7168 <-> 3584 projections,
RMSNorm on the aggregate and two fused shared experts; LATENT below):

  latent_tiny   6 tokens, hidden 512 around the tiny experts (latent 256), shared 256
  latent1       1 token, hidden 7168 around the decode1 experts, shared 2 x 3072
  latent32      32 tokens, hidden 7168 around the prefill32 experts, shared 2 x 3072

Dense weights are bf16 values: w_down ~ N(0, 1/Dh), w_up ~ N(0, 1/Dl), shared
gate/up ~ N(0, 1/Dh), shared down ~ N(0, 1/Fs), norm weight 1 + 0.1 N(0, 1), so
every stage stays O(1); hidden states h ~ N(0, 1) (bf16 values) and the router
logits are h . R with R ~ N(0, 1/Dh) (the router reads the full hidden state).

Weights: each packed byte is drawn uniform over 0..255, i.e. both e2m1 nibbles
independent and uniform over the 16 codes.  Scale bytes are uniform integers over
an inclusive range.  Every (expert, tensor) pair has its own PCG64 sub-stream
``default_rng([weight_seed, expert, tensor_id])`` so any expert can be
regenerated alone (the oracle needs only the experts a sample touches).
tensor_id order: gate_q, gate_s, up_q, up_s, down_q, down_s.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

TENSORS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    E: int
    K: int
    D: int
    F: int
    weight_seed: int
    act_seed: int
    scale_lo: int
    scale_hi: int
    x_kind: str            # "normal" (i.i.d. N(0,1)) or "ar1"
    logit_kind: str        # "normal" (i.i.d. N(0,1)) or "hR" (h_t . R)
    bias_std: float        # score-correction bias ~ N(0, bias_std^2); 0 -> zeros
    path: str              # "decode" or "chunk"
    edge_experts: Tuple[int, ...] = ()
    x_bf16: bool = False   # hidden states rounded to bf16 (a workload with bf16 activations)
    edge_mode: str = "finite"  # "finite" or "literal" (see the module docstring)

    @property
    def pairs(self) -> int:
        return self.T * self.K

    def expert_bytes(self) -> int:
        """MXFP4 bytes of one expert: three [rows, cols/2] packed + [rows, cols/32] scales."""
        per = self.F * self.D // 2 + self.F * self.D // 32
        return 3 * per

    def shapes(self) -> Dict[str, Tuple[int, int]]:
        D, F = self.D, self.F
        return {
            "gate_q": (F, D // 2), "gate_s": (F, D // 32),
            "up_q": (F, D // 2), "up_s": (F, D // 32),
            "down_q": (D, F // 2), "down_s": (D, F // 32),
        }


_EDGE = tuple(range(0, 896, 112))  # 0, 112, ..., 784

CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", T=1, E=8, K=2, D=256, F=128, weight_seed=101, act_seed=101,
                   scale_lo=120, scale_hi=130, x_kind="normal", logit_kind="normal",
                   bias_std=0.1, path="decode"),
    "decode1": Config("decode1", T=1, E=896, K=16, D=3584, F=3072, weight_seed=102, act_seed=102,
                      scale_lo=118, scale_hi=128, x_kind="normal", logit_kind="normal",
                      bias_std=0.1, path="decode"),
    "prefill32": Config("prefill32", T=32, E=896, K=16, D=3584, F=3072, weight_seed=102,
                        act_seed=103, scale_lo=118, scale_hi=128, x_kind="ar1",
                        logit_kind="hR", bias_std=0.0, path="chunk"),
    "prefill256": Config("prefill256", T=256, E=896, K=16, D=3584, F=3072, weight_seed=102,
                         act_seed=104, scale_lo=118, scale_hi=128, x_kind="ar1",
                         logit_kind="hR", bias_std=0.0, path="chunk", x_bf16=True),
    "batch4096": Config("batch4096", T=4096, E=896, K=16, D=3584, F=3072, weight_seed=105,
                        act_seed=105, scale_lo=118, scale_hi=128, x_kind="normal",
                        logit_kind="hR", bias_std=0.0, path="chunk", edge_experts=_EDGE),
}


def scaled(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller T, other E/D/F ...)."""
    return dataclasses.replace(cfg, **changes)


# ----------------------------------------------------------------------------- weights
EDGE_FRACTION = 0.25   # share of an edge expert's groups with a full-range scale byte
EDGE_ZERO_ABOVE = 128  # edge groups with a larger scale byte hold +-0 codes only


def _tensor(cfg: Config, e: int, tid: int) -> np.ndarray:
    name = TENSORS[tid]
    shape = cfg.shapes()[name]
    rng = np.random.default_rng([cfg.weight_seed, e, tid])
    edge = e in cfg.edge_experts
    if name.endswith("_q"):
        q = rng.integers(0, 256, size=shape, dtype=np.uint8)
        if edge and cfg.edge_mode == "finite":
            s = _tensor(cfg, e, tid + 1)  # the scale bytes of the same rows
            zero = np.repeat(s > EDGE_ZERO_ABOVE, 16, axis=1)  # 16 packed bytes per group
            q = np.where(zero, q & 0x88, q).astype(np.uint8)
        return q
    if edge and cfg.edge_mode == "literal":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    s = rng.integers(cfg.scale_lo, cfg.scale_hi + 1, size=shape, dtype=np.uint8)
    if edge:
        pick = rng.random(shape) < EDGE_FRACTION
        s = np.where(pick, rng.integers(0, 256, size=shape, dtype=np.uint8), s).astype(np.uint8)
    return s


def expert_tensors(cfg: Config, e: int) -> Dict[str, np.ndarray]:
    """The six MXFP4 tensors of expert ``e`` (host numpy uint8)."""
    if not 0 <= e < cfg.E:
        raise ValueError(f"expert {e} out of range for E={cfg.E}")
    return {name: _tensor(cfg, e, tid) for tid, name in enumerate(TENSORS)}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def weights_host(cfg: Config, experts: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """Stacked host weights ``{name: [n, rows, cols]}`` for ``experts`` (default: all)."""
    ids = list(range(cfg.E)) if experts is None else [int(e) for e in experts]
    out = {n: np.empty((len(ids),) + cfg.shapes()[n], dtype=np.uint8) for n in TENSORS}

    def fill(j_e):
        j, e = j_e
        for tid, n in enumerate(TENSORS):
            out[n][j] = _tensor(cfg, e, tid)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, enumerate(ids)))
    return out


def weights_device(cfg: Config, device, batch: int = 32, experts: Optional[Iterable[int]] = None):
    """Experts as torch uint8 tensors ``{name: [E, rows, cols]}`` on ``device``.

    All E experts by default; with ``experts`` only those are generated and the
    others are left zero (for short runs that touch a known subset).  Generated on
    the host in batches of ``batch`` experts and copied up, so the host never
    holds more than one batch.
    """
    import torch

    alloc = torch.empty if experts is None else torch.zeros
    dev = {n: alloc((cfg.E,) + cfg.shapes()[n], dtype=torch.uint8, device=device) for n in TENSORS}
    ids_all = list(range(cfg.E)) if experts is None else sorted({int(e) for e in experts})
    for b0 in range(0, len(ids_all), batch):
        ids = ids_all[b0:b0 + batch]
        host = weights_host(cfg, ids)
        for n in TENSORS:
            src = torch.from_numpy(host[n])
            if ids == list(range(ids[0], ids[0] + len(ids))):
                dev[n][ids[0]:ids[0] + len(ids)].copy_(src, non_blocking=False)
            else:
                for j, e in enumerate(ids):
                    dev[n][e].copy_(src[j], non_blocking=False)
    return dev


# ------------------------------------------------------------------------- activations
def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), returned as fp32.

    The bf16-activation workload's hidden states are these values; both the
    oracle and the device receive exactly them."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).reshape(np.shape(x))


def activations(cfg: Config, T: Optional[int] = None, stream: int = 0, bf16: Optional[bool] = None):
    """``(x [T,D] f32, logits [T,E] f32, bias [E] f32)`` for the workload.

    ``stream`` selects an independent draw of the same distribution (used to
    build several different decode tokens for cache-cold timing).  For a
    workload with bf16 activations (``cfg.x_bf16``, or ``bf16=True``) the hidden
    states are bf16 values held in fp32, and the logits are computed from those
    values.
    """
    bf16 = cfg.x_bf16 if bf16 is None else bf16
    T = cfg.T if T is None else int(T)
    rng = np.random.default_rng([cfg.act_seed, 7919, stream])
    if cfg.x_kind == "normal":
        x64 = rng.standard_normal((T, cfg.D))
    elif cfg.x_kind == "ar1":
        # h_t = 0.9 h_{t-1} + 0.436 z_t, started at the stationary law h_0 ~ N(0, I)
        z = rng.standard_normal((T, cfg.D))
        x64 = np.empty_like(z)
        x64[0] = z[0]
        for t in range(1, T):
            x64[t] = 0.9 * x64[t - 1] + 0.436 * z[t]
    else:
        raise ValueError(cfg.x_kind)
    x = x64.astype(np.float32)
    if bf16:
        x = bf16_round(x)

    if cfg.logit_kind == "normal":
        logits = rng.standard_normal((T, cfg.E)).astype(np.float32)
    elif cfg.logit_kind == "hR":
        # R ~ N(0, variance 1/D), so logits = h.R are ~N(0, 1) per entry
        R = np.random.default_rng([cfg.act_seed, 104729]).standard_normal((cfg.D, cfg.E))
        R *= np.sqrt(1.0 / cfg.D)
        logits = (x.astype(np.float64) @ R).astype(np.float32)
    else:
        raise ValueError(cfg.logit_kind)

    if cfg.bias_std > 0:
        bias = (cfg.bias_std * np.random.default_rng([cfg.act_seed, 31337]).standard_normal(cfg.E)
                ).astype(np.float32)
    else:
        bias = np.zeros(cfg.E, dtype=np.float32)
    return np.ascontiguousarray(x), np.ascontiguousarray(logits), bias


def sample_tokens(cfg: Config, n: int, must_include: Sequence[int] = (), seed: int = 0) -> np.ndarray:
    """A sorted, seeded sample of ``n`` token ids plus every id in ``must_include``."""
    rng = np.random.default_rng([cfg.act_seed, 271828, seed])
    base = rng.choice(cfg.T, size=min(n, cfg.T), replace=False)
    return np.unique(np.concatenate([base, np.asarray(must_include, dtype=np.int64)])).astype(np.int64)


# --------------------------------------------------------------------- LatentMoE block
@dataclasses.dataclass(frozen=True)
class LatentConfig:
    name: str
    experts: Config        # the routed experts (their D is the latent width)
    Dh: int                # hidden width
    Fs: int                # width of the two fused shared experts (both halves)
    seed: int
    eps: float = 1e-6


LATENT: Dict[str, LatentConfig] = {
    "latent_tiny": LatentConfig("latent_tiny", scaled(CONFIGS["tiny"], T=6, path="chunk"), Dh=512, Fs=256, seed=501),
    "latent1": LatentConfig("latent1", CONFIGS["decode1"], Dh=7168, Fs=6144, seed=502),
    "latent32": LatentConfig("latent32", CONFIGS["prefill32"], Dh=7168, Fs=6144, seed=503),
}

DENSE = ("w_down", "w_up", "norm", "shared_gate", "shared_up", "shared_down")


def latent_dense_host(lc: LatentConfig) -> Dict[str, np.ndarray]:
    """The dense weights of a LatentMoE block as bf16 values held in fp32."""
    Dh, Dl, Fs = lc.Dh, lc.experts.D, lc.Fs
    shapes = {"w_down": (Dl, Dh), "w_up": (Dh, Dl), "norm": (Dl,), "shared_gate": (Fs, Dh),
              "shared_up": (Fs, Dh), "shared_down": (Dh, Fs)}
    std = {"w_down": Dh ** -0.5, "w_up": Dl ** -0.5, "shared_gate": Dh ** -0.5, "shared_up": Dh ** -0.5,
           "shared_down": Fs ** -0.5}
    out = {}
    for tid, n in enumerate(DENSE):
        rng = np.random.default_rng([lc.seed, 4242, tid])
        if n == "norm":
            v = 1.0 + 0.1 * rng.standard_normal(shapes[n])
        else:
            v = std[n] * rng.standard_normal(shapes[n], dtype=np.float32)
        out[n] = bf16_round(np.asarray(v, dtype=np.float32))
    return out


def latent_activations(lc: LatentConfig, T: Optional[int] = None):
    """``(h [T,Dh] bf16 values in f32, logits [T,E] f32, bias [E] f32)``."""
    cfg = lc.experts
    T = cfg.T if T is None else int(T)
    rng = np.random.default_rng([lc.seed, 7919])
    h = bf16_round(rng.standard_normal((T, lc.Dh)).astype(np.float32))
    R = np.random.default_rng([lc.seed, 104729]).standard_normal((lc.Dh, cfg.E)) * np.sqrt(1.0 / lc.Dh)
    logits = (h.astype(np.float64) @ R).astype(np.float32)
    if cfg.bias_std > 0:
        bias = (cfg.bias_std * np.random.default_rng([lc.seed, 31337]).standard_normal(cfg.E)).astype(np.float32)
    else:
        bias = np.zeros(cfg.E, dtype=np.float32)
    return np.ascontiguousarray(h), np.ascontiguousarray(logits), bias
