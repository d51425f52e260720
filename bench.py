"""Benchmark of the MI355X routed-expert block (one GPU).

A step is one pass of the block's hot path for one decode token at the K3 shape
(896 experts, top-16, D=3584, F=3072, MXFP4): the router on the token's logits,
then the 16 selected experts' gate/up GEMVs, SiTU-GLU, down GEMVs and the
weighted combine.  Steps rotate over 32 pre-generated tokens whose expert sets
differ, so each step streams its 16 experts (280.76 MB) from HBM rather than from
the 256 MB last-level cache.  The value is routed-expert weight bytes per second
over the timed steps (inputs resident in HBM).

Also reported: the 4096-token chunk pass (grouped bf16-MFMA path, and the
MXFP8-activation path on the scaled FP8 x FP4 MFMA with one and two parts) in TFLOP/s,
the roofline of the decode gate/up kernel from HIP events that its launch records at
the kernel's start and end, and the CPU oracle timed on a bounded sample as a
baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import statistics
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-expert MXFP4 GB/s + µs/layer-token (decode); TFLOP/s (chunk) vs roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0  # dense FP8 (and FP8 x FP4 scaled) MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# counter summaries per kind, and the sources whose change invalidates them
TRAFFIC_FILES = {"decode": os.path.join("profiles", "decode_gateup_traffic.json"),
                 "chunk": os.path.join("profiles", "chunk_gemm_traffic.json")}
TRAFFIC_SOURCES = {
    "decode": ("mxfp4_routed_expert_k3moe_amd/csrc/decode.hip", "mxfp4_routed_expert_k3moe_amd/csrc/device.hpp",
               "mxfp4_routed_expert_k3moe_amd/csrc/launch.hpp"),
    "chunk": ("mxfp4_routed_expert_k3moe_amd/csrc/chunk.hip", "mxfp4_routed_expert_k3moe_amd/csrc/gemm.hpp",
              "mxfp4_routed_expert_k3moe_amd/csrc/device.hpp", "mxfp4_routed_expert_k3moe_amd/csrc/launch.hpp")}
PROBE_TOKENS = 8
COPY_BYTES = 1 << 30


def sources_digest(kind: str = "decode") -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(kind: str = "decode"):
    """The committed counter summary of `kind`, or None when it is missing or was
    taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILES[kind])
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    return t if t.get("sources_sha256") == sources_digest(kind) else None


def traffic_bytes():
    """HBM bytes per decode gate/up launch from the committed counter runs, or None."""
    t = traffic_record("decode")
    return None if t is None else t.get("bytes_per_launch")


def tokens_per_expert(lib, idx, E):
    """Min / median / max of the tokens routed to each expert of the union, from the
    library's own grouping (k3moe_group)."""
    counts = lib.group(idx, E)["counts"].cpu().numpy()
    used = counts[counts > 0]
    return {"min": int(used.min()), "median": float(np.median(used)), "max": int(used.max())}


def capture_steps(torch, fn, n):
    """A HIP graph (torch.cuda.CUDAGraph) of the n calls fn(0) .. fn(n-1), captured
    on a side stream of default priority.  Every call's kernels are replayed with
    the call's own inputs; only the host-side launch work leaves the timed region."""
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


def timed_steps(torch, fn, n, extra=0):
    """Seconds for the n calls fn(0) .. fn(n-1): one HIP graph replay (after an
    untimed one), or, if capture fails on this machine, the n calls issued eagerly
    between two synchronizations.  `extra` more timed repetitions follow the first
    (replays, or eager passes) for the spread.  Returns (seconds, mode, [seconds of
    each extra repetition])."""
    try:
        g = capture_steps(torch, fn, n)
    except RuntimeError as exc:
        torch.cuda.synchronize()
        log(f"graph capture failed ({exc}); timing eagerly")
        times = []
        for _ in range(1 + extra):
            t0 = time.perf_counter()
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        return times[0], "eager", times[1:]
    el = timed_replay(torch, g)
    more = []
    for _ in range(extra):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        WALL.append(time.perf_counter() - t0)
        more.append(e0.elapsed_time(e1) * 1e-3)
    del g
    return el, "graph", more


def timed_replay(torch, g):
    """One untimed replay (the first one uploads the graph), then one timed replay
    between two synchronizations; returns seconds of GPU time (events recorded on
    the stream around the replay) and records the host clock's reading of the same
    bracket in WALL."""
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    WALL.append(time.perf_counter() - t0)
    return e0.elapsed_time(e1) * 1e-3


WALL = []  # host-clock seconds of each timed replay, in order


def chunk_algorithmic_bytes(cfg, U, T):
    """Algorithmic HBM bytes of the two grouped GEMM launches of one fp32 chunk pass:
    gate/up reads the union's gate and up tensors and x once as 16-bit values (the
    fp16 items read x in fp16; the few items on the bf16 path read its high part and
    low part instead) and writes h (16-bit, one row per pair); down reads the down
    tensors and h and writes the per-pair fp32 rows."""
    P = T * cfg.K
    tensor = cfg.F * cfg.D // 2 + cfg.F * cfg.D // 32
    gate_up = U * 2 * tensor + T * cfg.D * 2 + P * cfg.F * 2
    down = U * tensor + P * cfg.F * 2 + P * cfg.D * 4
    return {"gemm_gateup": gate_up, "gemm_down": down}


def counters_probe_chunk(torch, synth, lib, dev):
    """A short run for rocprofv3 --pmc: the 4096-token fp32 chunk pass twice, then a
    plain device copy of COPY_BYTES twice (the calibration)."""
    cfg = synth.CONFIGS["batch4096"]
    W = lib.ExpertWeights.from_dict(synth.weights_device(cfg, dev))
    x, lg, bs = synth.activations(cfg)
    xc = torch.from_numpy(x).to(dev)
    idx, w = lib.route(torch.from_numpy(lg).to(dev), torch.from_numpy(bs).to(dev), cfg.K)
    ws = torch.empty(lib.workspace_size(lib.OP_CHUNK, cfg.T, cfg.K, W), dtype=torch.uint8, device=dev)
    for _ in range(2):
        lib.forward_chunk(W, xc, idx, w, ws=ws)
    a = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"chunk counters probe: 2 passes of {cfg.T} tokens, copy {COPY_BYTES} B x 2")


def counters_probe(torch, synth, lib, dev):
    """A short run for rocprofv3 --pmc: PROBE_TOKENS decode tokens through route,
    gate/up and down (only the experts they touch are generated), then a plain
    device copy of COPY_BYTES twice, whose counter readings calibrate the bytes."""
    cfg = synth.CONFIGS["decode1"]
    xs, logits, bias = synth.activations(cfg, T=PROBE_TOKENS, stream=5)
    l_d, b_d = torch.from_numpy(logits).to(dev), torch.from_numpy(bias).to(dev)
    idx, w = lib.route(l_d, b_d, cfg.K)
    used = np.unique(idx.cpu().numpy())
    W = lib.ExpertWeights.from_dict(synth.weights_device(cfg, dev, experts=used))
    x_d = torch.from_numpy(xs).to(dev)
    y = torch.empty((PROBE_TOKENS, cfg.D), dtype=torch.float32, device=dev)
    ws = torch.empty(lib.workspace_size(lib.OP_DECODE, 1, cfg.K, W), dtype=torch.uint8, device=dev)
    for j in range(PROBE_TOKENS):
        lib.forward_decode(W, x_d[j], idx[j], w[j], y=y[j], ws=ws)
    a = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"counters probe: {PROBE_TOKENS} tokens, {len(used)} experts, copy {COPY_BYTES} B x 2")


def _pmc_rows(folder, counter):
    """(kernel name, value in bytes) per dispatch from a rocprofv3 csv folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))  # KiB -> B
    return rows


def _calibrated(rows, match, counter):
    """Mean calibrated bytes per dispatch of the kernels whose name contains `match`."""
    copy = [v for n, v in rows if "copy" in n.lower() and v > COPY_BYTES / 4]
    ks = [v for n, v in rows if match in n]
    if not copy or not ks:
        raise SystemExit(f"{counter}: copy dispatches {len(copy)}, {match} dispatches {len(ks)}")
    factor = COPY_BYTES / float(np.median(copy))
    return {"counter": counter, "raw_bytes_per_launch": float(np.mean(ks)), "copy_raw_bytes": float(np.median(copy)),
            "calibration_factor": factor, "bytes_per_launch": float(np.mean(ks)) * factor, "launches": len(ks)}


def summarize_counters(fetch_dir, write_dir, kind="decode"):
    if kind == "decode":
        cfg_k, cfg_f, cfg_d = 16, 3072, 3584
        algo = cfg_k * 2 * (cfg_f * cfg_d // 2 + cfg_f * cfg_d // 32) + cfg_d * 4 + cfg_k * cfg_f * 4
        kernels = {"decode_gateup_kernel": ("decode_gateup_kernel", algo)}
    else:
        import synth
        cfg = synth.CONFIGS["batch4096"]
        algos = chunk_algorithmic_bytes(cfg, cfg.E, cfg.T)  # the 4096-token union is all 896 experts
        kernels = {"gemm_gateup": ("gemm_kernel<0,", algos["gemm_gateup"]), "gemm_down": ("gemm_kernel<1,", algos["gemm_down"])}
    out = {"kind": kind, "sources_sha256": sources_digest(kind), "copy_bytes": COPY_BYTES, "kernels": {}}
    rows = {"fetch": _pmc_rows(fetch_dir, "FETCH_SIZE"), "write": _pmc_rows(write_dir, "WRITE_SIZE")}
    for name, (match, algo) in kernels.items():
        rows_n = {k: [(n.replace(" ", ""), v) for n, v in r] for k, r in rows.items()}
        per = {key: _calibrated(rows_n[key], match.replace(" ", ""), cnt)
               for key, cnt in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"))}
        tot = round(per["fetch"]["bytes_per_launch"] + per["write"]["bytes_per_launch"])
        out["kernels"][name] = dict(per, algorithmic_bytes_per_launch=algo, bytes_per_launch=tot,
                                    traffic_over_algorithmic=round(tot / algo, 4))
    if kind == "decode":  # flat fields read by the bench line
        k = out["kernels"]["decode_gateup_kernel"]
        out.update(kernel="decode_gateup_kernel", algorithmic_bytes_per_launch=k["algorithmic_bytes_per_launch"],
                   bytes_per_launch=k["bytes_per_launch"], traffic_over_algorithmic=k["traffic_over_algorithmic"])
    with open(os.path.join(ROOT, TRAFFIC_FILES[kind]), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def achievable_peaks(torch, lib, dev):
    """Rates the library's probe kernels reach on this GPU, beside the published
    peaks: a streaming read of a 2 GiB buffer (best over loads in flight per thread
    and plain or non-temporal loads), the same over 281 MB (one decode token's
    expert bytes, so ramp-up and drain count as they do for the decode kernels),
    and MFMA issue loops (bf16 16x16x32; scaled 16x16x128 FP8 x FP4, FP4 x FP4)."""
    stream = torch.cuda.current_stream()
    out = {}
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)

    def rate(nbytes, unroll, nt, blocks, reps):
        view = buf[:nbytes]
        lib.probe_stream_read(view, unroll, nt, blocks, sink=sink)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib.probe_stream_read(view, unroll, nt, blocks, sink=sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return nbytes / (statistics.median(ts) * 1e-3) / 1e9

    best = (0.0, None)
    for unroll in (4, 8, 16):
        for nt in (False, True):
            for blocks in (2048, 4096, 8192):
                g = rate(2 << 30, unroll, nt, blocks, 5)
                if g > best[0]:
                    best = (g, {"unroll": unroll, "nontemporal": nt, "blocks": blocks})
    out["hbm_read_gbs"] = round(best[0], 1)
    out["hbm_read_config"] = best[1]
    small = 280756224 // 16 * 16
    out["hbm_read_281MB_gbs"] = round(max(rate(small, best[1]["unroll"], best[1]["nontemporal"], b, 20)
                                          for b in (1024, 2048, 4096)), 1)
    del buf
    flops = {0: 16384, 1: 65536, 2: 65536, 4: 32768, 5: 131072, 6: 131072}
    names = {0: "bf16_16x16x32", 1: "fp8_fp4_16x16x128", 2: "fp4_fp4_16x16x128", 4: "bf16_32x32x16",
             5: "fp4_fp4_32x32x64", 6: "fp8_fp4_32x32x64"}
    blocks, iters = 2048, 2000
    o = torch.empty(4 * blocks, dtype=torch.float32, device=dev)
    for kind in (0, 4, 1, 6, 2, 5):
        lib.probe_mfma(kind, 10, blocks, out=o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.probe_mfma(kind, iters, blocks, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out[f"mfma_{names[kind]}_tflops"] = round(blocks * 4 * iters * 8 * flops[kind] / (ms * 1e-3) / 1e12, 1)
    log(f"achievable: read {out['hbm_read_gbs']:.0f} GB/s ({best[1]}), 281 MB {out['hbm_read_281MB_gbs']:.0f} GB/s; "
        "MFMA TFLOP/s " + ", ".join(f"{k[5:-7]} {v:.0f}" for k, v in out.items() if k.startswith("mfma_")))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--chunk-iters", type=int, default=10)
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-latent", action="store_true", help="skip the LatentMoE block legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--top-p", type=float, default=0.7, help="also time decode with top-p pruning (0 = skip)")
    ap.add_argument("--pool-slots", type=int, default=128,
                    help="also time decode with experts in pinned host memory behind an HBM pool (0 = skip)")
    ap.add_argument("--counters-probe", nargs="?", const="decode", choices=("decode", "chunk"),
                    help="run only a few decode steps (or two 4096-token chunk passes) and the copy calibration "
                         "(for rocprofv3 --pmc)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders into the counter summary of --kind")
    ap.add_argument("--kind", default="decode", choices=("decode", "chunk"))
    ap.add_argument("--replays", type=int, default=0,
                    help="extra timed replays of the K-step graph for the spread (default: enough for >= 50 steps)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, kind=args.kind)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this block's kernels run on a single MI355X "
              "(multi-GPU sharding is a design note, not implemented); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from mxfp4_routed_expert_k3moe_amd import lib

    lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.counters_probe == "decode":
        counters_probe(torch, synth, lib, dev)
        return
    if args.counters_probe == "chunk":
        counters_probe_chunk(torch, synth, lib, dev)
        return

    # ------------------------------------------------------------- decode workload
    cfg = synth.CONFIGS["decode1"]
    log(f"generating {cfg.name} weights ({cfg.E} experts, {cfg.E * cfg.expert_bytes() / 1e9:.1f} GB)")
    t0 = time.time()
    W = lib.ExpertWeights.from_dict(synth.weights_device(cfg, dev))
    log(f"weights resident in {time.time() - t0:.1f}s")
    n_rot = 32
    xs, logits, bias = synth.activations(cfg, T=n_rot, stream=5)
    x_d = torch.from_numpy(xs).to(dev)
    l_d = torch.from_numpy(logits).to(dev)
    b_d = torch.from_numpy(bias).to(dev)
    K = cfg.K
    idx_d = torch.empty((n_rot, K), dtype=torch.int32, device=dev)
    w_d = torch.empty((n_rot, K), dtype=torch.float32, device=dev)
    y_d = torch.empty((n_rot, cfg.D), dtype=torch.float32, device=dev)
    ws = torch.empty(lib.workspace_size(lib.OP_DECODE, 1, K, W), dtype=torch.uint8, device=dev)
    bytes_per_token = K * cfg.expert_bytes()  # 280 756 224

    def step(j, ev=None):
        # the router kernel on the token's logits, then forward_decode (gate/up +
        # SiTU-GLU, down, combine); on a bracketed step the gate/up launch records a
        # pair of events at the kernel's start and end
        lib.route(l_d[j:j + 1], b_d, K, idx=idx_d[j:j + 1], w=w_d[j:j + 1])
        if ev is None:
            lib.forward_decode(W, x_d[j], idx_d[j], w_d[j], y=y_d[j], ws=ws)
        else:
            lib.forward_decode_timed(W, x_d[j], idx_d[j], w_d[j], ev[0].cuda_event, ev[1].cuda_event, y=y_d[j], ws=ws)

    for i in range(args.warmup):
        step(i % n_rot)
    torch.cuda.synchronize()
    y_ref = y_d.clone()  # eager outputs of the 32 tokens (the warm-up covers each at least once)
    if args.warmup < n_rot:
        for j in range(n_rot):
            step(j)
        torch.cuda.synchronize()
        y_ref = y_d.clone()

    # timed region: exactly `steps` steps (token i % 32 at step i), captured as one
    # HIP graph and replayed between two synchronizations after an untimed replay
    y_d.zero_()
    extra = args.replays if args.replays > 0 else max(4, -(-50 // args.steps))
    n_wall = len(WALL)
    elapsed, mode, more = timed_steps(torch, lambda i: step(i % n_rot), args.steps, extra)
    wall = np.array(WALL[n_wall:]) * 1e3 / args.steps  # host-clock ms per step of the same replays
    # the tokens the timed steps ran (all 32 once K >= 32) against their eager outputs
    n_chk = min(args.steps, n_rot)
    replay_ok = bool(torch.equal(y_d[:n_chk].view(torch.int32), y_ref[:n_chk].view(torch.int32)))
    ms_per_step = elapsed * 1e3 / args.steps
    value = bytes_per_token * args.steps / elapsed / 1e9
    spread = np.array([elapsed] + more) * 1e3 / args.steps  # ms per step of every timed repetition
    log(f"decode: {mode} timing of {args.steps} steps, outputs of {n_chk} tokens equal to the eager ones: {replay_ok}; "
        f"{len(spread)} repetitions: median {np.median(spread) * 1e3:.1f} us/step "
        f"(p10 {np.percentile(spread, 10) * 1e3:.1f}, p90 {np.percentile(spread, 90) * 1e3:.1f})")

    # the gate/up kernel's own duration: eager steps whose gate/up launch records a
    # pair of events at the kernel's start and end (hipExtLaunchKernelGGL; each event
    # is recorded once beforehand so that its HIP event exists)
    n_ev = min(max(args.steps, 1), 64)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(n_ev):
        step(i % n_rot, evs[i])
    torch.cuda.synchronize()
    gu_ms = np.array([a.elapsed_time(b) for a, b in evs])  # gate/up kernel per bracketed call
    gu_avg_us = float(np.mean(gu_ms) * 1e3)
    # algorithmic bytes of one gate/up launch: 16 experts' gate and up tensors, x in, h out
    gu_bytes = K * 2 * (cfg.F * cfg.D // 2 + cfg.F * cfg.D // 32) + cfg.D * 4 + K * cfg.F * 4
    achieved = gu_bytes / (gu_avg_us * 1e-6) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step (route + gate/up + down + combine), gate/up kernel {gu_avg_us:.1f} us "
        f"(p10 {np.percentile(gu_ms, 10) * 1e3:.1f}, p90 {np.percentile(gu_ms, 90) * 1e3:.1f}) -> "
        f"{achieved:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode1: 1 token/step (rotating over 32), 896 experts top-16, D=3584, F=3072, "
                               "MXFP4 experts, fp32 activations",
                   "tokens_per_step": 1, "experts": cfg.E, "top_k": K, "d_model": cfg.D, "d_ff": cfg.F,
                   "expert_bytes_per_token": bytes_per_token},
        "us_per_layer_token": round(ms_per_step * 1e3, 3),
        "timing": {"mode": ("the K steps captured as one HIP graph, one untimed replay, then one timed replay"
                            if mode == "graph" else "the K steps issued eagerly (graph capture failed)"),
                   "clock": ("GPU time between events recorded on the stream around each replay, with a "
                             "device synchronization before and after" if mode == "graph" else "host clock"),
                   "wall_us_per_step_first": round(float(wall[0]) * 1e3, 3) if len(wall) else None,
                   "wall_us_per_step_median": round(float(np.median(wall)) * 1e3, 3) if len(wall) else None,
                   "replay_outputs_equal_eager": replay_ok, "replay_tokens_checked": n_chk,
                   "repetitions": len(spread), "steps_timed_in_all": len(spread) * args.steps,
                   "us_per_step_median": round(float(np.median(spread)) * 1e3, 3),
                   "us_per_step_p10": round(float(np.percentile(spread, 10)) * 1e3, 3),
                   "us_per_step_p90": round(float(np.percentile(spread, 90)) * 1e3, 3),
                   "gateup_kernel_us_p10": round(float(np.percentile(gu_ms, 10)) * 1e3, 3),
                   "gateup_kernel_us_p90": round(float(np.percentile(gu_ms, 90)) * 1e3, 3)},
        "roofline": {"bound": "hbm", "kernel": "decode_gateup_kernel (16 experts' gate/up GEMV + SiTU-GLU)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_bytes(),
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_avg_us, 3)},
    }

    # top-p pruning (colibri PR #676, K3_TOPP paragraph) on the same tokens: the
    # router drops the low-weight tail and the decode kernels skip pruned slots
    top_p = args.top_p
    if top_p > 0.0:
        n_kept = torch.empty(1, dtype=torch.int32, device=dev)
        kept_all = []
        for j in range(n_rot):
            lib.route_topp(l_d[j:j + 1], b_d, K, top_p, idx=idx_d[j:j + 1], w=w_d[j:j + 1], n_kept=n_kept)
            kept_all.append(int(n_kept.item()))

        def step_topp(j):
            lib.route_topp(l_d[j:j + 1], b_d, K, top_p, idx=idx_d[j:j + 1], w=w_d[j:j + 1], n_kept=n_kept)
            lib.forward_decode(W, x_d[j], idx_d[j], w_d[j], y=y_d[j], ws=ws)

        for i in range(args.warmup):
            step_topp(i % n_rot)
        torch.cuda.synchronize()
        el, _, _ = timed_steps(torch, lambda i: step_topp(i % n_rot), args.steps)
        kept_mean = float(np.mean([kept_all[i % n_rot] for i in range(args.steps)]))
        us = el * 1e6 / args.steps
        result["decode_topp"] = {"top_p": top_p, "mean_experts_kept": round(kept_mean, 3), "of": K,
                                 "us_per_layer_token": round(us, 3),
                                 "kept_expert_gbs": round(kept_mean * cfg.expert_bytes() / us / 1e3, 1),
                                 "speedup_vs_top16": round(ms_per_step * 1e3 / us, 3)}
        log(f"decode top-p {top_p}: {kept_mean:.2f} of {K} experts kept, {us:.1f} us/step")

    # expert residency (colibri PR #676, It runs the full model; PR #684 engine
    # commit): the layer's experts live in pinned host memory in the slot layout,
    # an LRU pool of HBM slots holds a subset, each token's misses are copied in
    # on a copy stream while its resident experts compute
    if args.pool_slots > 0:
        layout = lib.slot_layout(cfg.D, cfg.F)
        host = torch.empty((cfg.E, layout[6]), dtype=torch.uint8, pin_memory=True)
        for ti, name in enumerate(lib.ExpertWeights.NAMES):
            src = W.tensors[name].reshape(cfg.E, -1)
            host[:, layout[ti]:layout[ti] + src.shape[1]].copy_(src)
        torch.cuda.synchronize()
        slots_mem = torch.empty(args.pool_slots * layout[6], dtype=torch.uint8, device=dev)
        pool = lib.Pool(args.pool_slots, cfg.D, cfg.F, slots_mem)
        copy_stream = torch.cuda.Stream()
        ws_p = torch.empty(lib.workspace_size(lib.OP_DECODE, 1, K, W) + 768, dtype=torch.uint8, device=dev)
        for j in range(n_rot):  # the plain routing again (the top-p leg rewrote idx/w)
            lib.route(l_d[j:j + 1], b_d, K, idx=idx_d[j:j + 1], w=w_d[j:j + 1])

        def step_pooled(j):
            lib.route(l_d[j:j + 1], b_d, K, idx=idx_d[j:j + 1], w=w_d[j:j + 1])
            lib.forward_decode_pooled(pool, 0, host, 0, host.stride(0), x_d[j], idx_d[j], w_d[j], y=y_d[j],
                                      ws=ws_p, copy_stream=copy_stream)

        n_pool = min(args.steps, 64)
        for i in range(min(args.warmup, 8)):
            step_pooled(i % n_rot)
        torch.cuda.synchronize()
        st0 = pool.stats()
        t0 = time.perf_counter()
        for i in range(n_pool):
            step_pooled(i % n_rot)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        st1 = pool.stats()
        miss = st1["misses"] - st0["misses"]
        hit = st1["hits"] - st0["hits"]
        copied = st1["bytes"] - st0["bytes"]
        result["decode_pooled"] = {"pool_slots": args.pool_slots, "pool_gb": round(args.pool_slots * layout[6] / 1e9, 2),
                                   "tokens": n_pool, "hit_rate": round(hit / max(1, hit + miss), 4),
                                   "us_per_layer_token": round(el * 1e6 / n_pool, 2),
                                   "host_to_hbm_gbs": round(copied / el / 1e9, 2),
                                   "resident_us_per_layer_token": round(ms_per_step * 1e3, 2)}
        log(f"decode pooled ({args.pool_slots} slots): hit rate {hit / max(1, hit + miss):.3f}, "
            f"{el * 1e6 / n_pool:.1f} us/token, host->HBM {copied / el / 1e9:.1f} GB/s")
        pool.close()
        del host, slots_mem, pool

    # the LatentMoE block around the same experts (colibri PR #684 engine commit,
    # Stable LatentMoE bullet): 7168 -> 3584 projection, the routed experts,
    # RMSNorm on the aggregate, 3584 -> 7168, plus the two fused shared experts
    if not args.no_latent:
        lc = synth.LATENT["latent1"]
        dense_h = synth.latent_dense_host(lc)
        Lw = lib.LatentWeights({k: torch.from_numpy(v).to(torch.bfloat16).to(dev) for k, v in dense_h.items()},
                               lc.eps)
        dense_bytes = sum(int(v.size) * 2 for v in dense_h.values())
        hs, lgs, bss = synth.latent_activations(lc, T=n_rot)
        h_l = torch.from_numpy(hs).to(torch.bfloat16).to(dev)
        idx_l, w_l = lib.route(torch.from_numpy(lgs).to(dev), torch.from_numpy(bss).to(dev), K)
        out_l = torch.empty((n_rot, lc.Dh), dtype=torch.float32, device=dev)
        ws_l = torch.empty(lib.load().k3moe_latent_workspace_size(Lw.ref(), 1, K, W.ref()), dtype=torch.uint8,
                           device=dev)
        for j in range(min(args.warmup, n_rot)):
            lib.latent_forward(Lw, W, h_l[j:j + 1], idx_l[j:j + 1], w_l[j:j + 1], out=out_l[j:j + 1], ws=ws_l)
        torch.cuda.synchronize()
        n_lat = min(args.steps, 64)
        el_lat, _, _ = timed_steps(torch, lambda i: lib.latent_forward(Lw, W, h_l[i % n_rot:i % n_rot + 1],
                                                                    idx_l[i % n_rot:i % n_rot + 1],
                                                                    w_l[i % n_rot:i % n_rot + 1],
                                                                    out=out_l[i % n_rot:i % n_rot + 1], ws=ws_l),
                                n_lat)
        us = el_lat * 1e6 / n_lat
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        T_c = 256
        hc, lgc, bsc = synth.latent_activations(lc, T=T_c)
        h_c = torch.from_numpy(hc).to(torch.bfloat16).to(dev)
        idx_cl, w_cl = lib.route(torch.from_numpy(lgc).to(dev), torch.from_numpy(bsc).to(dev), K)
        out_c = torch.empty((T_c, lc.Dh), dtype=torch.float32, device=dev)
        ws_c = torch.empty(lib.load().k3moe_latent_workspace_size(Lw.ref(), T_c, K, W.ref()), dtype=torch.uint8,
                           device=dev)
        lib.latent_forward(Lw, W, h_c, idx_cl, w_cl, out=out_c, ws=ws_c)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.chunk_iters):
            lib.latent_forward(Lw, W, h_c, idx_cl, w_cl, out=out_c, ws=ws_c)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_c = e0.elapsed_time(e1) / args.chunk_iters
        result["latent"] = {"workload": f"LatentMoE block: hidden {lc.Dh}, the decode1 experts in the {cfg.D} latent, "
                                        f"RMSNorm, shared experts of width {lc.Fs} (bf16 dense weights)",
                            "decode_us_per_layer_token": round(us, 2),
                            "decode_weight_gbs": round((bytes_per_token + dense_bytes) / us / 1e3, 1),
                            "chunk256_ms": round(ms_c, 4), "chunk256_us_per_layer_token": round(ms_c * 1e3 / T_c, 3)}
        log(f"latent block: {us:.1f} us/token at T=1, {ms_c:.3f} ms for {T_c} tokens")
        del Lw, ws_l, ws_c
    # prefill chunks of 32 and 256 tokens on the same weight set (AR(1) hidden
    # states, logits = h.R): the grouped path streams each expert of the chunk's
    # union once, so the expert bytes per token fall by P / U (the pages observe
    # about 2.7x on real text at 32 tokens)
    if not args.no_chunk:
        result["prefill"] = {}
        for name in ("prefill32", "prefill256"):
            pc = synth.CONFIGS[name]
            x, lg, bs = synth.activations(pc)
            xp = torch.from_numpy(x).to(dev)
            if pc.x_bf16:  # the 256-token workload's bf16 activations (x holds bf16 values: exact)
                xp = xp.to(torch.bfloat16)
            lg_p, bs_p = torch.from_numpy(lg).to(dev), torch.from_numpy(bs).to(dev)
            idx_p, w_p = lib.route(lg_p, bs_p, pc.K)
            yp = torch.empty((pc.T, pc.D), dtype=torch.float32, device=dev)
            nu = torch.zeros(1, dtype=torch.int32, device=dev)
            wsp = torch.empty(lib.workspace_size(lib.OP_CHUNK, pc.T, pc.K, W), dtype=torch.uint8, device=dev)
            lib.forward_chunk(W, xp, idx_p, w_p, y=yp, n_unique=nu, ws=wsp)
            torch.cuda.synchronize()
            iters = 20 if pc.T <= 32 else 10
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                lib.route(lg_p, bs_p, pc.K, idx=idx_p, w=w_p)
                lib.forward_chunk(W, xp, idx_p, w_p, y=yp, n_unique=nu, ws=wsp)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            U, P = int(nu.item()), pc.T * pc.K
            result["prefill"][name] = {
                "tokens": pc.T, "ms": round(ms, 4), "us_per_layer_token": round(ms * 1e3 / pc.T, 3),
                "unique_experts": U, "pairs": P, "dedup": round(P / U, 3),
                "expert_bytes_per_token": round(U * cfg.expert_bytes() / pc.T),
                "weight_gbs": round(U * cfg.expert_bytes() / ms / 1e6, 1),
                "tflops": round(6.0 * pc.D * pc.F * P / ms / 1e9, 2),
                "tokens_per_expert": tokens_per_expert(lib, idx_p, pc.E)}
            log(f"{name}: {ms:.3f} ms ({ms * 1e3 / pc.T:.1f} us/layer-token), union {U} of {P} pairs "
                f"(dedup {P / U:.2f}x), {U * cfg.expert_bytes() / ms / 1e6:.0f} GB/s of expert weights")
            del wsp
    del W, ws
    torch.cuda.empty_cache()

    # -------------------------------------------------------------- chunk workload
    chunk_outputs, chunk_sample = {}, None
    if not args.no_chunk:
        ccfg = synth.CONFIGS["batch4096"]
        log(f"generating {ccfg.name} weights")
        Wc = lib.ExpertWeights.from_dict(synth.weights_device(ccfg, dev))
        x, lg, bs = synth.activations(ccfg)
        xc = torch.from_numpy(x).to(dev)  # fp32 hidden states
        lg_c, bs_c = torch.from_numpy(lg).to(dev), torch.from_numpy(bs).to(dev)
        idx_c, w_c = lib.route(lg_c, bs_c, ccfg.K)
        yc = torch.empty((ccfg.T, ccfg.D), dtype=torch.float32, device=dev)
        nu = torch.zeros(1, dtype=torch.int32, device=dev)
        flops = 6.0 * ccfg.D * ccfg.F * ccfg.T * ccfg.K
        # 16 seeded tokens whose outputs the CPU leg checks against the oracle
        chunk_sample = np.sort(np.random.default_rng(4096).choice(ccfg.T, 16, replace=False))
        chunk_outputs = {}

        def time_passes(fn):
            """Per-pass milliseconds of `chunk_iters` passes (route + fn), each
            between its own pair of events, after one untimed pass."""
            lib.route(lg_c, bs_c, ccfg.K, idx=idx_c, w=w_c)
            fn()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.chunk_iters)]
            for a, b in evs:
                a.record(stream)
                lib.route(lg_c, bs_c, ccfg.K, idx=idx_c, w=w_c)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in evs])

        def leg(ms_all, U, extra=None):
            ms = float(np.median(ms_all))
            wbytes = U * ccfg.expert_bytes()
            d = {"ms": round(ms, 4), "ms_p10": round(float(np.percentile(ms_all, 10)), 4),
                 "ms_p90": round(float(np.percentile(ms_all, 90)), 4), "passes": len(ms_all),
                 "us_per_layer_token": round(ms * 1e3 / ccfg.T, 4), "tflops": round(flops / ms / 1e9, 2),
                 # fp16 and bf16 dense MFMA share one peak (the items run on either)
                 "tflops_frac_16bit_peak": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                 "peak_tflops": BF16_PEAK_TFLOPS,
                 "weight_gbs": round(wbytes / ms / 1e6, 1)}
            d.update(extra or {})
            return d

        wsc = torch.empty(lib.workspace_size(lib.OP_CHUNK, ccfg.T, ccfg.K, Wc), dtype=torch.uint8, device=dev)
        ms_all = time_passes(lambda: lib.forward_chunk(Wc, xc, idx_c, w_c, y=yc, n_unique=nu, ws=wsc))
        U = int(nu.item())
        chunk_outputs["chunk"] = yc[torch.from_numpy(chunk_sample).to(dev)].cpu().numpy()
        tr = traffic_record("chunk")
        result["chunk"] = leg(ms_all, U, {
            "workload": "batch4096: 4096 tokens, i.i.d. fp32 hidden states, logits = h.R, same shape, grouped MFMA "
                        "GEMMs: fp16 (x and h in fp16) on items whose weights are fp16 normals, bf16 with the MXFP4 "
                        "low part of x elsewhere (route + group + split + gate/up + down + combine)",
            "unique_experts": U, "tokens_per_expert": tokens_per_expert(lib, idx_c, ccfg.E),
            "traffic": None if tr is None else {k: {"bytes_per_launch": v["bytes_per_launch"],
                                                    "algorithmic_bytes_per_launch": v["algorithmic_bytes_per_launch"],
                                                    "traffic_over_algorithmic": v["traffic_over_algorithmic"]}
                                                for k, v in tr["kernels"].items()}})
        log(f"chunk: {result['chunk']['ms']:.3f} ms (p10 {result['chunk']['ms_p10']:.3f}, p90 "
            f"{result['chunk']['ms_p90']:.3f}), {result['chunk']['tflops']:.1f} TFLOP/s, union {U}")
        del wsc
        torch.cuda.empty_cache()
        # the same pass with MXFP8 activations on the scaled FP8 x FP4 MFMA, one and two parts
        wsm = torch.empty(lib.workspace_size(lib.OP_CHUNK_MX, ccfg.T, ccfg.K, Wc), dtype=torch.uint8, device=dev)
        result["chunk_mx"] = {"workload": "batch4096 as above, MXFP8 activations (E4M3 + E8M0 per 32) in one or "
                                          "two parts, scaled FP8 x FP4 MFMA (route + group + quantize + gate/up + "
                                          "down + combine); a lower-precision variant, its distance to the exact "
                                          "block is in cpu_baseline.accuracy"}
        for parts in (1, 2):
            ms_all = time_passes(lambda: lib.forward_chunk_mx(Wc, xc, idx_c, w_c, parts, y=yc, n_unique=nu, ws=wsm))
            chunk_outputs[f"chunk_mx_parts{parts}"] = yc[torch.from_numpy(chunk_sample).to(dev)].cpu().numpy()
            d = leg(ms_all, U)
            d["tflops_frac_fp8_peak"] = round(d["tflops"] / FP8_PEAK_TFLOPS, 4)
            result["chunk_mx"][f"parts{parts}"] = d
            log(f"chunk mx parts={parts}: {d['ms']:.3f} ms, {d['tflops']:.1f} TFLOP/s")
        del Wc, wsm
        torch.cuda.empty_cache()

    # achievable peaks last: their 2 GiB probe buffer must not shape the legs above
    torch.cuda.empty_cache()
    peaks = achievable_peaks(torch, lib, dev)
    torch.cuda.empty_cache()
    result["achievable_peaks"] = peaks
    result["roofline"]["frac_of_achievable_read"] = round(result["roofline"]["achieved"] / peaks["hbm_read_gbs"], 4)

    # ---------------------------------------------------------------- CPU baseline
    # the oracle (plain C, double sums) on this host: the decode workload on the
    # box's CPU share (16 threads for one GPU), one thread for the tiny and decode
    # workloads, the near-tie count of each workload's routing, and the chunk legs'
    # sampled outputs against the exact block
    if not args.no_cpu:
        import platform
        import oracle
        n_thr = 16
        try:
            cpu_model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        except (OSError, StopIteration):
            cpu_model = platform.processor()
        xs_h, lg_h, bs_h = synth.activations(cfg, T=160, stream=9)
        idx_h, w_h, _ = oracle.route(lg_h, bs_h, K)

        def decode_tokens(nthreads, budget_s, max_tokens):
            done, t_cpu = 0, 0.0
            while done < max_tokens and t_cpu < budget_s:
                used = np.unique(idx_h[done])
                Wh = synth.weights_host(cfg, used)
                local = np.searchsorted(used, idx_h[done:done + 1]).astype(np.int32)
                t0 = time.perf_counter()
                oracle.forward(Wh, xs_h[done:done + 1], local, w_h[done:done + 1], nthreads=nthreads)
                t_cpu += time.perf_counter() - t0
                done += 1
            return done, t_cpu

        done, t_cpu = decode_tokens(n_thr, args.cpu_seconds, 160)
        cpu_gbs = done * bytes_per_token / t_cpu / 1e9
        done1, t1 = decode_tokens(1, 6.0, 4)
        tiny = synth.CONFIGS["tiny"]
        Wt = synth.weights_host(tiny)
        xt, lgt, bst = synth.activations(tiny, T=256, stream=3)
        it, wt, _ = oracle.route(lgt, bst, tiny.K)
        t0 = time.perf_counter()
        oracle.forward(Wt, xt, it, wt, nthreads=1)
        t_tiny = (time.perf_counter() - t0) / xt.shape[0]
        near = {}
        for name in ("decode1", "prefill32", "prefill256", "batch4096"):
            c = synth.CONFIGS[name]
            _, lgn, bsn = synth.activations(c, T=32 if name == "decode1" else None, stream=5 if name == "decode1" else 0)
            _, _, gap = oracle.route(lgn, bsn, c.K)
            near[name] = {"tokens": int(gap.size), "gap_below_1e-6": int(np.count_nonzero(gap < 1e-6))}
        accuracy = {}
        if chunk_outputs:
            ccfg = synth.CONFIGS["batch4096"]
            x_s, lg_s, bs_s = synth.activations(ccfg)
            i_s, w_s, _ = oracle.route(lg_s[chunk_sample], bs_s, ccfg.K)
            used = np.unique(i_s)
            Ws = synth.weights_host(ccfg, used)
            loc = np.searchsorted(used, i_s).astype(np.int32)
            exact = oracle.forward(Ws, x_s[chunk_sample], loc, w_s, nthreads=n_thr).astype(np.float64)
            for k, got in chunk_outputs.items():
                accuracy[k] = float(np.linalg.norm(got - exact) / np.linalg.norm(exact))
        result["cpu_baseline"] = {
            "value": round(cpu_gbs, 4), "unit": "GB/s", "cores": n_thr, "kind": "oracle",
            "sample": f"{done} decode1 tokens (16 experts each, route excluded), {t_cpu:.1f} s on {n_thr} threads "
                      f"(the box's CPU share for one GPU)",
            "us_per_layer_token": round(t_cpu / done * 1e6, 1),
            "host": {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": cpu_model},
            "one_thread": {"decode1_us_per_layer_token": round(t1 / done1 * 1e6, 1), "decode1_tokens": done1,
                           "decode1_gbs": round(done1 * bytes_per_token / t1 / 1e9, 4),
                           "tiny_us_per_token": round(t_tiny * 1e6, 2)},
            "near_ties": near,
            "accuracy": {"what": "rel-L2 of 16 seeded tokens of each 4096-token leg against the exact block "
                                 "(the oracle on the fp32 hidden states)", **{k: round(v, 6) for k, v in accuracy.items()}}}
        log(f"cpu oracle: {cpu_gbs:.3f} GB/s over {done} tokens on {n_thr} threads; one thread "
            f"{t1 / done1 * 1e3:.0f} ms/token; near ties {near}; accuracy {accuracy}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
