"""Shared pieces of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys
import time
from typing import Dict, Optional

import numpy as np
import pytest

import oracle
import synth

_weights_cache: Dict[tuple, object] = {}


def timing_event():
    """A timing-enabled torch event whose HIP event already exists (recorded once),
    so its raw handle (``.cuda_event``) can be handed to a timed entry point."""
    torch = torch_cuda()
    ev = torch.cuda.Event(enable_timing=True)
    ev.record()
    return ev


def log(msg: str):
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_k3moe_amd import lib
    lib.load()  # raises if the HIP library is missing: no fallback
    return torch


def device_weights(cfg: synth.Config):
    """All experts of ``cfg`` on cuda:0 (cached per weight set)."""
    torch = torch_cuda()
    from mxfp4_routed_expert_k3moe_amd import lib
    key = (cfg.weight_seed, cfg.E, cfg.D, cfg.F, cfg.scale_lo, cfg.scale_hi, cfg.edge_experts)
    if key not in _weights_cache:
        if len(_weights_cache) >= 2:  # keep at most two big weight sets resident
            _weights_cache.pop(next(iter(_weights_cache)))
            torch.cuda.empty_cache()
        log(f"generating weights for {cfg.name} (E={cfg.E} D={cfg.D} F={cfg.F})")
        t0 = time.time()
        d = synth.weights_device(cfg, "cuda:0")
        _weights_cache[key] = lib.ExpertWeights.from_dict(d)
        log(f"weights ready in {time.time() - t0:.1f}s")
    return _weights_cache[key]


def oracle_forward_subset(cfg: synth.Config, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                          want_pairs: bool = False, mx: int = 0, weights=None, progress: int = 0):
    """The oracle on ``x [T,D]`` with routing ``idx/w [T,K]``, given host weights of
    only the experts the routing touches (regenerated from the seeded generator,
    or taken from ``weights`` when given).  ``mx`` selects the MXFP8 variant;
    ``progress=n`` has the oracle report every n-th finished expert."""
    used = np.unique(idx[idx >= 0])  # pruned slots (id -1) touch no expert
    if weights is None:
        log(f"oracle: generating {len(used)} experts' weights")
        W = synth.weights_host(cfg, used)
    else:
        W = {k: v[used] for k, v in weights.items()}
    local = np.where(idx >= 0, np.searchsorted(used, np.maximum(idx, 0)), -1).astype(np.int32)
    t0 = time.time()
    out = oracle.forward(W, x, local, w, want_pairs=want_pairs, mx=mx, progress=progress)
    if progress:
        log(f"oracle: {x.shape[0]} tokens, {len(used)} experts in {time.time() - t0:.1f}s")
    return out


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    """||got - want|| / ||want|| in float64 over elements finite in both."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(want, dtype=np.float64).ravel()
    ok = np.isfinite(g) & np.isfinite(r)
    den = np.linalg.norm(r[ok])
    return float(np.linalg.norm(g[ok] - r[ok]) / den) if den > 0 else float(np.linalg.norm(g[ok]))


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str, per_token: Optional[int] = None):
    """Non-finite masks (NaN and +-inf as one class) must agree, and the rel-L2
    over elements finite in both must be within ``tol``."""
    g = np.asarray(got)
    r = np.asarray(want)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    mg, mr = ~np.isfinite(g), ~np.isfinite(r)
    n_bad = int(np.count_nonzero(mg != mr))
    assert n_bad == 0, f"{what}: non-finite masks differ at {n_bad} elements"
    e = rel_l2(g, r)
    log(f"{what}: rel-L2 {e:.3e} (tol {tol:g}), non-finite {int(mr.sum())}")
    assert e <= tol, f"{what}: rel-L2 {e:.3e} > {tol:g}"
    return e
