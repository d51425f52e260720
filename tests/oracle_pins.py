"""Pins that tie the CPU oracle to what the pages and mathematics fix.

Each ``check_*`` takes an oracle instance (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees.  ``test_oracle_pins.py`` runs them on
the oracle as built; ``test_oracle_mutations.py`` runs them on copies of the
oracle with one planted mistake each and requires that some check fails.

None of these checks retypes the oracle's code: decode is compared with a value
set derived from the e2m1 bit fields in exact rationals, the layout with a
hand-worked fixture, sums with exact rational brute force, the activation with
40-digit decimal arithmetic and its SwiGLU limit, the router with brute-force
subset search, invariants and a case that separates the two readings of where
the bias goes.
"""
from __future__ import annotations

import itertools
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- reference helpers
def e2m1_value(code: int) -> Fraction:
    """e2m1 from its bit fields: sign bit3, exponent bits 2..1 (bias 1), mantissa bit0;
    exponent field 0 is subnormal (m * 0.5)."""
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if code & 8 else mag


def fp32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def closed_form_bits(code: int, s: int) -> int:
    """fp32 bits of v * 2^(s-127), rounded to nearest (exact below 2^128, else inf)."""
    v = e2m1_value(code)
    mag = abs(v) * Fraction(2) ** (s - 127)
    if mag >= 2 ** 128:
        bits = 0x7F800000
    else:
        f = float(mag)
        assert Fraction(f) == mag  # at most two significant bits: exact in double
        bits = fp32_bits(f)
        assert Fraction(struct.unpack("<f", struct.pack("<I", bits))[0]) == mag  # and in fp32
    return bits | (0x80000000 if code & 8 else 0)


def f32_bits_array(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


getcontext().prec = 40


def _dexp(x) -> Decimal:
    return Decimal(x).exp()


def _dtanh(x) -> Decimal:
    x = Decimal(x)
    e2 = (2 * x).exp()
    return (e2 - 1) / (e2 + 1)


def _dsig(x) -> Decimal:
    return 1 / (1 + _dexp(-Decimal(x)))


def situ_decimal(g, u) -> Decimal:
    """K3's SiTU-GLU at betas 4 and 25 in 40-digit decimal arithmetic."""
    g, u = Decimal(repr(float(g))), Decimal(repr(float(u)))
    return 4 * _dtanh(g / 4) * _dsig(g) * 25 * _dtanh(u / 25)


def layout_fixture():
    rows = []
    with open(os.path.join(HERE, "golden", "mxfp4_layout.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            b, s, v0, v1 = line.split()
            conv = lambda t: float.fromhex(t) if "0x" in t else float(t)
            rows.append((int(b, 16), int(s), conv(v0), conv(v1)))
    return rows


# ------------------------------------------------------------------------ P1 decode
def check_decode_closed_form(o):
    """All 16 codes x 256 scale bytes equal the closed form, bit for bit."""
    table = f32_bits_array(o.decode_table())
    for c in range(16):
        for s in range(256):
            want = closed_form_bits(c, s)
            got = int(table.reshape(16, 256)[c, s])
            assert got == want, f"decode(code={c}, s={s}): {got:#010x} != {want:#010x}"
    # doubled e2m1 values are exact int8 (int8-activation commit, colibri PR #684)
    for c in range(16):
        d = 2 * e2m1_value(c)
        assert d.denominator == 1 and -128 <= d.numerator <= 127


def check_decode_conventions(o):
    """The edge readings stated in the design: subnormals kept at s=0, s=255 is the
    closed form (not NaN), code 8 is -0.0."""
    assert fp32_bits(o.decode(1, 0)) == 0x00200000          # 0.5 * 2^-127 = 2^-128
    assert fp32_bits(o.decode(7, 0)) == fp32_bits(1.5 * 2.0 ** -125)
    assert fp32_bits(o.decode(0, 255)) == 0x00000000
    assert fp32_bits(o.decode(8, 255)) == 0x80000000
    assert fp32_bits(o.decode(1, 255)) == 0x7F000000        # 2^127
    assert fp32_bits(o.decode(9, 255)) == 0xFF000000
    assert fp32_bits(o.decode(2, 255)) == 0x7F800000        # 2^128 -> +inf
    assert fp32_bits(o.decode(10, 255)) == 0xFF800000
    for s in range(256):
        assert fp32_bits(o.decode(8, s)) == 0x80000000


# ------------------------------------------------------------------------ P2 layout
def check_layout_fixture(o):
    for byte, s, v_even, v_odd in layout_fixture():
        q = np.full((1, 16), byte, dtype=np.uint8)
        sc = np.full((1, 1), s, dtype=np.uint8)
        out = o.dequant(q, sc)
        for i in range(32):
            want = v_even if i % 2 == 0 else v_odd
            assert fp32_bits(float(out[0, i])) == fp32_bits(want), (hex(byte), s, i, out[0, i], want)


def check_scale_groups(o):
    """A scale byte applies to its own 32 columns only, and each row to its own scales."""
    q = np.full((2, 32), 0x22, dtype=np.uint8)          # every code = 2 -> v = 1.0
    s = np.array([[127, 129], [125, 127]], dtype=np.uint8)
    out = o.dequant(q, s)
    assert np.all(out[0, :32] == 1.0) and np.all(out[0, 32:] == 4.0)
    assert np.all(out[1, :32] == 0.25) and np.all(out[1, 32:] == 1.0)


def check_dequant_matches_codes(o):
    """Random matrix: element (o, i) is the closed form of its own nibble and scale."""
    rng = np.random.default_rng(11)
    O, I = 3, 96
    q = rng.integers(0, 256, size=(O, I // 2), dtype=np.uint8)
    s = rng.integers(0, 256, size=(O, I // 32), dtype=np.uint8)
    got = f32_bits_array(o.dequant(q, s))
    for r in range(O):
        for i in range(I):
            byte = int(q[r, i // 2])
            code = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
            assert int(got[r, i]) == closed_form_bits(code, int(s[r, i // 32])), (r, i)


# ------------------------------------------------------------------------ P3 matmul
def check_expert_brute_force(o):
    """A 4 x 64 expert: g, u and y equal exact rational sums (relative 1e-12)."""
    rng = np.random.default_rng(3)
    D, F = 64, 4
    Wg = rng.standard_normal((F, D)).astype(np.float32)
    Wu = rng.standard_normal((F, D)).astype(np.float32)
    Wd = rng.standard_normal((D, F)).astype(np.float32)
    x = rng.standard_normal(D).astype(np.float32)
    r = o.expert(Wg, Wu, Wd, x)
    for name, W in (("g", Wg), ("u", Wu)):
        for f in range(F):
            exact = sum(Fraction(float(W[f, i])) * Fraction(float(x[i])) for i in range(D))
            scale = sum(abs(Fraction(float(W[f, i])) * Fraction(float(x[i]))) for i in range(D))
            assert abs(Fraction(r[name][f]) - exact) <= Fraction(1, 10 ** 12) * scale, (name, f)
    for f in range(F):
        assert r["h"][f] == o.situ(r["g"][f], r["u"][f])
    for d in range(D):
        exact = sum(Fraction(float(Wd[d, f])) * Fraction(float(r["h"][f])) for f in range(F))
        scale = sum(abs(Fraction(float(Wd[d, f])) * Fraction(float(r["h"][f]))) for f in range(F))
        assert abs(Fraction(r["y"][d]) - exact) <= Fraction(1, 10 ** 12) * scale + Fraction(1, 10 ** 300), d


# ------------------------------------------------------------------------- P4 route
def _brute_topk(keys, K):
    """All K-subsets whose every member beats every non-member (ties -> lower id)."""
    E = len(keys)
    better = lambda a, b: keys[a] > keys[b] or (keys[a] == keys[b] and a < b)
    sols = [S for S in itertools.combinations(range(E), K)
            if all(better(a, b) for a in S for b in range(E) if b not in S)]
    assert len(sols) == 1
    return set(sols[0])


def check_route_brute_force(o):
    """E=8, K=2: the selection is the unique subset that dominates the rest, listed
    in descending key order; weights sum to one."""
    rng = np.random.default_rng(17)
    for trial in range(20):
        logits = rng.standard_normal((1, 8)).astype(np.float32)
        bias = (0.1 * rng.standard_normal(8)).astype(np.float32)
        idx, w, gap = o.route(logits, bias, 2)
        # keys rebuilt with a textbook sigmoid in decimal, rounded to fp32, plus the bias
        keys = [np.float32(np.float32(float(_dsig(Decimal(repr(float(l)))))) + bias[e])
                for e, l in enumerate(logits[0])]
        assert set(idx[0].tolist()) == _brute_topk(keys, 2), trial
        assert keys[idx[0, 0]] > keys[idx[0, 1]] or (keys[idx[0, 0]] == keys[idx[0, 1]] and idx[0, 0] < idx[0, 1])
        assert abs(float(w.sum(dtype=np.float64)) - 1.0) <= 2 * 2.0 ** -24
        sel = sorted(keys, reverse=True)
        assert abs(gap[0] - (float(sel[1]) - float(sel[2]))) <= 1e-12


def check_route_invariants(o):
    rng = np.random.default_rng(23)
    T, E, K = 16, 896, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    idx, w, gap = o.route(logits, bias, K)
    for t in range(T):
        assert len(set(idx[t].tolist())) == K
        assert abs(float(w[t].sum(dtype=np.float64)) - 1.0) <= K * 2.0 ** -24
        assert np.all(w[t] > 0)
    # zero bias: selection is the top-K logits (sigmoid is monotone)
    idx0, w0, _ = o.route(logits, np.zeros(E, np.float32), K)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        assert set(idx0[t].tolist()) == set(order[:K]), t
    # weights depend on the selection only, not on the bias (they renormalize the raw sigmoid scores):
    # lowering the bias of unselected experts keeps every selected key and the selection
    for t in range(T):
        b2 = bias.copy()
        mask = np.ones(E, bool)
        mask[idx[t]] = False
        b2[mask] -= np.float32(1.0)
        idx1, w1, _ = o.route(logits[t:t + 1], b2, K)
        assert np.array_equal(idx1[0], idx[t]) and np.array_equal(w1[0], w[t]), t
    # K = 1: weight exactly 1; equal logits: weights exactly 1/K, ties to lower ids
    idxk, wk, _ = o.route(logits[:1], bias, 1)
    assert wk[0, 0] == 1.0
    flat = np.zeros((1, 10), np.float32)
    idxf, wf, _ = o.route(flat, np.zeros(10, np.float32), 4)
    assert idxf[0].tolist() == [0, 1, 2, 3] and np.all(wf == np.float32(0.25))
    # K = E: w_e = sigma(l_e) / sum sigma, checked in decimal
    l = rng.standard_normal((1, 6)).astype(np.float32)
    idxa, wa, _ = o.route(l, np.zeros(6, np.float32), 6)
    sig = [_dsig(Decimal(repr(float(v)))) for v in l[0]]
    tot = sum(sig)
    for k in range(6):
        want = float(sig[idxa[0, k]] / tot)
        assert abs(float(wa[0, k]) - want) <= 2.0 ** -24 * want


def check_route_bias_reading(o):
    """The bias corrects the SCORE sigma(l)+b, not the logit: l=(0,4), b=(0.5,0)
    selects expert 0 (1.0 > 0.982), while sigma(l+b) would select expert 1."""
    idx, w, _ = o.route(np.array([[0.0, 4.0]], np.float32), np.array([0.5, 0.0], np.float32), 1)
    assert idx[0, 0] == 0 and w[0, 0] == 1.0
    idx, w, _ = o.route(np.array([[0.0, 4.0, -1.0]], np.float32), np.array([0.5, 0.0, 0.0], np.float32), 2)
    assert idx[0].tolist() == [0, 1]
    s0, s1 = 1 / (1 + math.exp(-0.0)), 1 / (1 + math.exp(-4.0))
    assert abs(float(w[0, 0]) - s0 / (s0 + s1)) <= 1e-7 and abs(float(w[0, 1]) - s1 / (s0 + s1)) <= 1e-7


def check_route_nan(o):
    """NaN logits rank below every number and are taken, lowest id first, only when
    fewer than K finite keys remain."""
    l = np.array([[np.nan, 1.0, np.nan, -2.0, np.nan]], np.float32)
    idx, _, _ = o.route(l, np.zeros(5, np.float32), 3)
    assert idx[0].tolist() == [1, 3, 0]


# -------------------------------------------------------------------------- P5 SiTU
def check_situ(o):
    pts = [(4.0, 25.0), (1.0, 4.0), (4.0, 1.0), (-3.0, 7.0), (0.5, -30.0), (10.0, 100.0),
           (-0.25, 0.125), (37.0, -61.0)]
    for g, u in pts:
        want = situ_decimal(g, u)
        got = o.situ(g, u)
        assert abs(Decimal(got) - want) <= Decimal("1e-14") * max(abs(want), Decimal("1e-300")), (g, u, got, want)
    for v in (0.0, 1.5, -7.0, 300.0):
        assert o.situ(0.0, v) == 0.0 and o.situ(v, 0.0) == 0.0
        assert o.situ(3.0, -v) == -o.situ(3.0, v)                      # odd in u
    for u in (1.0, -12.0, 40.0):
        assert abs(o.situ(1e4, u) - 100.0 * math.tanh(u / 25.0)) <= 1e-13 * 100
        assert o.situ(-1e4, u) == 0.0 and o.situ(-math.inf, u) == 0.0
        assert abs(o.situ(math.inf, u) - 100.0 * math.tanh(u / 25.0)) <= 1e-13
        assert math.isnan(o.situ(math.nan, u)) and math.isnan(o.situ(u, math.nan))
    lim = 25.0 * 4.0 * math.tanh(0.5) / (1.0 + math.exp(-2.0))
    assert abs(o.situ(2.0, math.inf) - lim) <= 1e-15 * lim
    # generic betas -> infinity give SwiGLU g * sigma(g) * u (textbook special case)
    for g, u in [(1.3, -0.7), (-2.0, 3.0), (0.25, 0.5)]:
        swiglu = float(Decimal(g) * _dsig(g) * Decimal(u))
        assert abs(o.situ_beta(g, u, 1e8, 1e8) - swiglu) <= 1e-9 * abs(swiglu)
    # the K3 form is the generic form at betas 4 and 25
    assert o.situ(2.5, -9.0) == o.situ_beta(2.5, -9.0, 4.0, 25.0)


# ------------------------------------------------------------- P6/P7 forward, combine
def _tiny():
    import synth
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=6)
    W = synth.weights_host(cfg)
    x, logits, bias = synth.activations(cfg)
    return cfg, W, x, logits, bias


def check_forward_pairs(o):
    """Pair (t,k) uses expert idx[t,k]'s decoded weights on token t's x; y_t is the
    w-weighted sum of its pairs in k order."""
    cfg, W, x, logits, bias = _tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    y, ytk, hk = o.forward(W, x, idx, w, nthreads=2, want_pairs=True)
    for t in range(cfg.T):
        for k in range(cfg.K):
            e = int(idx[t, k])
            Wg = o.dequant(W["gate_q"][e], W["gate_s"][e])
            Wu = o.dequant(W["up_q"][e], W["up_s"][e])
            Wd = o.dequant(W["down_q"][e], W["down_s"][e])
            r = o.expert(Wg, Wu, Wd, x[t])
            assert np.array_equal(ytk[t, k], r["y"]) and np.array_equal(hk[t, k], r["h"]), (t, k)
        acc = np.zeros(cfg.D)
        for k in range(cfg.K):
            acc = acc + np.float64(w[t, k]) * ytk[t, k]
        assert np.array_equal(y[t], acc.astype(np.float32)), t


def check_forward_combine(o):
    cfg, W, x, logits, bias = _tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    y = o.forward(W, x, idx, w, nthreads=2)
    # linear in w (doubling is exact)
    y2 = o.forward(W, x, idx, 2 * w, nthreads=2)
    assert np.array_equal(y2, 2 * y)
    # K = 1, w = 1: the single expert's output
    e = int(idx[0, 0])
    y1 = o.forward(W, x[:1], idx[:1, :1], np.ones((1, 1), np.float32), nthreads=1)
    r = o.expert(o.dequant(W["gate_q"][e], W["gate_s"][e]), o.dequant(W["up_q"][e], W["up_s"][e]),
                 o.dequant(W["down_q"][e], W["down_s"][e]), x[0])
    assert np.array_equal(y1[0], r["y"].astype(np.float32))


def check_chunk_equals_tokens(o):
    """A chunk's output is bit-identical to running its tokens one at a time (the
    chunked-prefill invariant, colibri PR #676 validation table)."""
    cfg, W, x, logits, bias = _tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    y = o.forward(W, x, idx, w, nthreads=3)
    for t in range(cfg.T):
        yt = o.forward(W, x[t:t + 1], idx[t:t + 1], w[t:t + 1], nthreads=1)
        assert np.array_equal(yt[0], y[t]), t


# -------------------------------------------------------------------------- P8 group
def check_group(o):
    rng = np.random.default_rng(29)
    for T, K, E in [(1, 2, 8), (7, 3, 5), (33, 16, 896), (64, 4, 9)]:
        idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
        g = o.group(idx, E)
        pairs = [(int(idx[p // K, p % K]), p) for p in range(T * K)]
        want_perm = [p for _, p in sorted(pairs)]
        assert g["perm"].tolist() == want_perm
        counts = [sum(1 for e, _ in pairs if e == x) for x in range(E)]
        assert g["counts"].tolist() == counts
        assert g["offsets"].tolist() == [sum(counts[:e]) for e in range(E + 1)]
        union = sorted(set(idx.ravel().tolist()))
        assert g["uniq"].tolist() == union and g["n_unique"] == len(union)


# -------------------------------------------------------------- P9 generator moments
def check_gate_moments(o):
    """std(g) over rows matches sqrt(D * E[w^2]) with E[w^2] = E[v^2] * mean(4^(s-127)),
    E[v^2] = 8.5625 over the 16 codes (1000+ rows, 3%)."""
    import synth
    cfg = synth.CONFIGS["decode1"]
    ex = synth.expert_tensors(cfg, 5)
    Wg = o.dequant(ex["gate_q"], ex["gate_s"])
    Wd = o.dequant(ex["down_q"], ex["down_s"])
    x = np.random.default_rng(1).standard_normal(cfg.D).astype(np.float32)
    g = o.expert(Wg, Wg, Wd, x)["g"]
    ev2 = float(sum(e2m1_value(c) ** 2 for c in range(16)) / 16)
    assert ev2 == 8.5625
    m4 = np.mean([4.0 ** (s - 127) for s in range(cfg.scale_lo, cfg.scale_hi + 1)])
    want = math.sqrt(cfg.D * ev2 * m4 * float(np.mean(x.astype(np.float64) ** 2)))
    got = float(np.sqrt(np.mean(g ** 2)))
    assert abs(got / want - 1) < 0.03, (got, want)


# ------------------------------------------------------------------- P10 top-p pruning
def _topp_exact(logits_row, bias_row, K, p):
    """The top-p rule ([PR676] K3_TOPP paragraph) in 40-digit decimal arithmetic on
    sigmoids computed here: selection by fp32 key as in the router, then the
    smallest weight-ordered prefix whose score sum reaches p of the total.  Returns
    (kept experts in slot order, their weights, decision margin)."""
    E = len(logits_row)
    sig = [_dsig(float(l)) for l in logits_row]
    keys = []
    for e in range(E):
        k = np.float32(np.float32(float(sig[e])) + np.float32(bias_row[e]))
        keys.append(-np.inf if np.isnan(k) else float(k))
    slots = sorted(range(E), key=lambda e: (-keys[e], e))[:K]
    S = sum(sig[e] for e in slots)
    order = sorted(range(K), key=lambda k: (-sig[slots[k]], k))
    thr = Decimal(repr(p)) * S
    cum, m, margin = Decimal(0), 0, None
    for r in order:
        cum += sig[slots[r]]
        m += 1
        margin = abs(cum - thr) / S if margin is None else min(margin, abs(cum - thr) / S)
        if cum >= thr:
            break
    kept_slots = sorted(order[:m])
    Sk = sum(sig[slots[k]] for k in kept_slots)
    return [slots[k] for k in kept_slots], [float(sig[slots[k]] / Sk) for k in kept_slots], margin


def check_route_topp_definition(o):
    """Kept experts = the smallest weight-ordered prefix of the top-K reaching p
    (the crossing expert kept), listed in slot order, renormalized over the kept
    raw scores; pruned slots hold id -1 and weight 0."""
    rng = np.random.default_rng(41)
    E, K, T = 32, 8, 24
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    skipped = 0
    for p in (0.3, 0.5, 0.7, 0.9):
        idx, w, n_kept, _ = o.route_topp(logits, bias, K, p)
        for t in range(T):
            want_ids, want_w, margin = _topp_exact(logits[t], bias, K, p)
            if margin < 1e-12:
                skipped += 1
                continue
            m = int(n_kept[t])
            assert m == len(want_ids) and 1 <= m <= K, (p, t)
            assert idx[t, :m].tolist() == want_ids, (p, t)
            assert np.all(idx[t, m:] == -1) and np.all(w[t, m:] == 0.0), (p, t)
            np.testing.assert_allclose(w[t, :m], want_w, rtol=1e-6, atol=0)
            assert abs(float(np.sum(w[t, :m], dtype=np.float64)) - 1.0) < 1e-6
    assert skipped < 4


def check_route_topp_off_and_monotone(o):
    """p outside (0, 1) prunes nothing (the plain router's output, bit for bit); the
    kept count never falls as p grows; p -> 0 keeps exactly the largest weight."""
    rng = np.random.default_rng(43)
    E, K, T = 48, 16, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    idx0, w0, _ = o.route(logits, bias, K)
    for p in (0.0, 1.0, 1.5, -0.2):
        idx, w, n_kept, _ = o.route_topp(logits, bias, K, p)
        assert np.array_equal(idx, idx0) and np.array_equal(w.view(np.uint32), w0.view(np.uint32))
        assert np.all(n_kept == K)
    prev = np.zeros(T, dtype=np.int32)
    for p in (1e-9, 0.2, 0.4, 0.6, 0.8, 0.95, 0.999):
        _, _, n_kept, _ = o.route_topp(logits, bias, K, p)
        assert np.all(n_kept >= prev)
        prev = n_kept
    idx, w, n_kept, _ = o.route_topp(logits, bias, K, 1e-9)
    assert np.all(n_kept == 1) and np.all(w[:, 0] == 1.0)
    sig = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    for t in range(T):
        assert idx[t, 0] == idx0[t][np.argmax(sig[t, idx0[t]])]


def check_forward_pruned(o):
    """A pruned slot (id -1) contributes nothing: the output equals the one with that
    slot routed to any expert at weight 0."""
    cfg, W, x, logits, bias = _tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    idx_p, w_p = idx.copy(), w.copy()
    idx_p[:, -1] = -1
    w_p[:, -1] = 0.0
    w_z = w.copy()
    w_z[:, -1] = 0.0
    assert np.array_equal(o.forward(W, x, idx_p, w_p), o.forward(W, x, idx, w_z))


def check_group_pruned(o):
    """Grouping skips pruned slots: counts, offsets and perm are those of the other pairs."""
    rng = np.random.default_rng(47)
    T, K, E = 19, 6, 11
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.3] = -1
    g = o.group(idx, E)
    pairs = [(int(idx[p // K, p % K]), p) for p in range(T * K) if idx[p // K, p % K] >= 0]
    assert g["perm"].tolist() == [p for _, p in sorted(pairs)]
    counts = [sum(1 for e, _ in pairs if e == x) for x in range(E)]
    assert g["counts"].tolist() == counts and int(g["offsets"][E]) == len(pairs)


# --------------------------------------------------------------- P10 MXFP8 activations
def e4m3_value(code: int):
    """OCP FP8 E4M3 from its bit fields: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN
    and there are no infinities.  Returns a Fraction, or None for NaN."""
    if code & 0x7F == 0x7F:
        return None
    e, m = (code >> 3) & 15, code & 7
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return -mag if code & 0x80 else mag


_E4M3_MAGS = [e4m3_value(c) for c in range(0x7F)]  # increasing in the code


def brute_mx_block(v):
    """One MX block of 32 fp32 values by search: the E8M0 scale is the s for which
    amax / 2^(s-127) lies in [256, 512) (so the largest value lands in E4M3's top
    binade), clamped to [0, 254]; each value goes to the nearest E4M3 magnitude after
    clamping to 448, ties to the even code, sign kept."""
    vals = [float(t) for t in v]
    if any(math.isnan(t) or math.isinf(t) for t in vals):
        return [0x7F] * 32, 255
    amax = max(Fraction(abs(t)) for t in vals)
    if amax == 0:
        return [0x80 if math.copysign(1.0, t) < 0 else 0 for t in vals], 0
    s = 0
    while s < 254 and amax >= 512 * Fraction(2) ** (s - 127):
        s += 1
    codes = []
    for t in vals:
        y = min(Fraction(abs(t)) / Fraction(2) ** (s - 127), Fraction(448))
        best = min(range(0x7F), key=lambda c: (abs(_E4M3_MAGS[c] - y), c & 1))
        codes.append(best | (0x80 if math.copysign(1.0, t) < 0 else 0))
    return codes, s


def mx_dequant_py(codes, s):
    return [float(e4m3_value(c) * Fraction(2) ** (s - 127)) for c in codes]


def check_e4m3_decode(o):
    """All 256 E4M3 codes decode to their bit-field values; the format's landmarks:
    448 largest finite, 2^-6 smallest normal, 2^-9 smallest subnormal."""
    for c in range(256):
        want, got = e4m3_value(c), o.e4m3(c)
        if want is None:
            assert math.isnan(got), c
        else:
            assert Fraction(got) == want, c
    assert o.e4m3(0x7E) == 448.0 and o.e4m3(0x08) == 2.0 ** -6 and o.e4m3(0x01) == 2.0 ** -9
    assert o.e4m3(0x38) == 1.0 and o.e4m3(0xB8) == -1.0


def check_mx_quant_exact_values(o):
    """A block whose largest magnitude is 448 has scale 2^0, and every E4M3 value in
    it is kept bit for bit (quantization is the inverse of decoding there)."""
    finite = [c for c in range(256) if c & 0x7F != 0x7F]
    blocks = []
    for i in range(0, len(finite), 31):
        part = finite[i:i + 31]
        part = part + [0] * (31 - len(part))
        blocks.append([0x7E] + part)
    val = lambda c: math.copysign(float(e4m3_value(c)), -1.0 if c & 0x80 else 1.0)  # keeps -0
    v = np.array([[val(c) for c in b] for b in blocks], np.float32)
    codes, scales = o.mx_quant(v.reshape(-1))
    assert scales.tolist() == [127] * len(blocks)
    assert codes.tolist() == [c for b in blocks for c in b]


def check_mx_quant_brute(o):
    """Random blocks over a wide spread of magnitudes, with exact ties, values past
    the saturation point and subnormal outputs: codes and scales equal the search."""
    rng = np.random.default_rng(53)
    blocks = []
    for b in range(48):
        v = rng.standard_normal(32) * np.exp2(rng.integers(-30, 30, size=32) * (b % 3 == 0))
        v *= 2.0 ** int(rng.integers(-95, 95))
        blocks.append(v)
    # ties: midpoints of adjacent E4M3 magnitudes under scale 2^0 (448 fixes the scale)
    mids = [float((_E4M3_MAGS[c] + _E4M3_MAGS[c + 1]) / 2) for c in range(0, 0x7E)]
    for i in range(0, len(mids), 31):
        part = mids[i:i + 31]
        blocks.append(np.array([448.0] + part + [0.0] * (31 - len(part))))
    # saturation: amax in (448, 512) times a power of two
    blocks.append(np.array([470.0, -500.0, 463.9, 464.0] + [1.0] * 28) * 2.0 ** 20)
    # tiny blocks: scale clamps at 0, subnormal fp32 inputs
    blocks.append(np.array([1e-39, -3e-40, 2e-45] + [0.0] * 29))
    blocks.append(np.array([-0.0] * 32))
    v = np.concatenate(blocks).astype(np.float32)
    codes, scales = o.mx_quant(v)
    for b in range(len(blocks)):
        want_c, want_s = brute_mx_block(v[32 * b:32 * b + 32])
        assert int(scales[b]) == want_s, (b, int(scales[b]), want_s)
        assert codes[32 * b:32 * b + 32].tolist() == want_c, b


def check_mx_quant_special(o):
    """Zero block: scale 0 and zero codes; a NaN or an infinity anywhere in a block
    makes the whole block NaN (E8M0 NaN scale 255, codes 0x7F), other blocks untouched."""
    v = np.zeros(128, np.float32)
    v[40] = np.nan
    v[64 + 3] = np.inf
    v[96:] = 1.0
    codes, scales = o.mx_quant(v)
    assert scales.tolist() == [0, 255, 255, 119]
    assert codes[:32].tolist() == [0] * 32 and codes[32:96].tolist() == [0x7F] * 64
    assert codes[96:].tolist() == [0x78] * 32  # 1.0 under scale 2^-8 is 256: exponent field 15


def brute_mx_parts(v, parts):
    """``parts`` MX parts by search: part 0 of v, then part 1 of the exact residual
    (which must be an fp32 value).  Returns the list of (codes, scale) and the
    exact value of the sum of the parts per element (None for NaN)."""
    c0, s0 = brute_mx_block(v)
    out = [(c0, s0)]
    vals = [None if s0 == 255 else e4m3_value(c) * Fraction(2) ** (s0 - 127) for c in c0]
    if parts == 2:
        res = []
        for t, q in zip(v, vals):
            r = float("nan") if q is None else Fraction(float(t)) - q
            if q is not None:
                assert Fraction(float(np.float32(float(r)))) == r  # the residual is exact in fp32
                r = float(r)
            res.append(r)
        c1, s1 = brute_mx_block(np.array(res, np.float32))
        out.append((c1, s1))
        vals = [None if (q is None or s1 == 255) else q + e4m3_value(c) * Fraction(2) ** (s1 - 127)
                for q, c in zip(vals, c1)]
    return out, vals


def check_mx_quant_two_parts(o):
    """Two parts: part 1 quantizes the exact residual of part 0; the sum of the two
    parts is within half a part-1 quantum of v (an error near 2^-8 of the block's
    largest magnitude instead of 2^-4)."""
    rng = np.random.default_rng(59)
    v = (rng.standard_normal(32 * 24) * np.exp2(rng.integers(-12, 12, size=32 * 24))).astype(np.float32)
    v[32 * 5:32 * 6] = 0.0
    v[32 * 7 + 3] = np.nan
    codes, scales = o.mx_quant(v, parts=2)
    assert codes.shape == (2, v.size) and scales.shape == (2, v.size // 32)
    for b in range(v.size // 32):
        blk = v[32 * b:32 * b + 32]
        parts, vals = brute_mx_parts(blk, 2)
        for pt in range(2):
            assert codes[pt, 32 * b:32 * b + 32].tolist() == parts[pt][0], (b, pt)
            assert int(scales[pt, b]) == parts[pt][1], (b, pt)
        if parts[0][1] != 255 and parts[0][1] > 0:
            amax = max(abs(Fraction(float(t))) for t in blk)
            for t, q in zip(blk, vals):
                assert abs(Fraction(float(t)) - q) <= amax * Fraction(1, 2 ** 7), b


def check_forward_mx(o):
    """The MXFP8 variant on a small block, one and two parts: every pair's h is the MX
    round trip of the fp32-rounded SiTU of exact sums over the MX round trip of x,
    and y is the exact w-weighted sum of the down rows over that h (fsum of exact
    products)."""
    import synth
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=2, E=4, K=2, D=64, F=64)
    W = synth.weights_host(cfg)
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = o.route(logits, bias, cfg.K)
    for parts in (1, 2):
        y, ytk, hk = o.forward(W, x, idx, w, nthreads=1, want_pairs=True, mx=parts)
        for t in range(cfg.T):
            xq = [float(q) for b in range(cfg.D // 32) for q in brute_mx_parts(x[t, 32 * b:32 * b + 32], parts)[1]]
            for k in range(cfg.K):
                e = int(idx[t, k])
                Wg = o.dequant(W["gate_q"][e], W["gate_s"][e]).astype(np.float64)
                Wu = o.dequant(W["up_q"][e], W["up_s"][e]).astype(np.float64)
                Wd = o.dequant(W["down_q"][e], W["down_s"][e]).astype(np.float64)
                hf = np.array([o.situ(math.fsum(Wg[f] * xq), math.fsum(Wu[f] * xq)) for f in range(cfg.F)],
                              np.float32)
                hq = [float(q) for b in range(cfg.F // 32) for q in brute_mx_parts(hf[32 * b:32 * b + 32], parts)[1]]
                assert np.allclose(hk[t, k], hq, rtol=2.0 ** -52, atol=0), (parts, t, k)
                for d in range(cfg.D):
                    terms = Wd[d] * np.array(hq)
                    exact = math.fsum(terms)
                    assert abs(ytk[t, k, d] - exact) <= 1e-12 * math.fsum(np.abs(terms)) + 1e-300, (parts, t, k, d)
            acc = np.zeros(cfg.D)
            for k in range(cfg.K):
                acc = acc + np.float64(w[t, k]) * ytk[t, k]
            assert np.array_equal(y[t], acc.astype(np.float32)), (parts, t)


def check_forward_mx_weight_scale_255(o):
    """The MX variant keeps the weights' closed form at scale byte 255 (w = v * 2^128,
    colibri PR #684, MXFP4-kernel commit): a down group of zero codes at s = 255 is
    +-0, so every output equals the one with that group's scale byte set to 127; and
    codes 1 / 9 (+-0.5) at s = 255 are the weights +-2^127, which codes 2 / 10
    (+-1.0) at s = 254 also denote, so those two encodings give identical outputs.
    Both hold for the exact path too."""
    import synth
    cfg = synth.scaled(synth.CONFIGS["tiny"], T=2, E=4, K=2, D=64, F=64)
    W = {k: v.copy() for k, v in synth.weights_host(cfg).items()}
    x, logits, bias = synth.activations(cfg)
    idx, w, _ = o.route(logits, bias, cfg.K)
    e = int(idx[0, 0])
    W["down_q"][e, 5, 0:16] = 0x80  # codes 0 and 8: +0 and -0
    W["down_s"][e, 5, 0] = 255
    W_ref = {k: v.copy() for k, v in W.items()}
    W_ref["down_s"][e, 5, 0] = 127
    # tiny weights beside a 2^127 group would vanish in h; the one-part MX h of
    # this block is O(1), so down products stay far below the fp32 range
    W_big = {k: v.copy() for k, v in W.items()}
    W_big["down_q"][e, 7, 16:32] = np.uint8(0x91)  # codes 1 and 9: +0.5, -0.5
    W_big["down_s"][e, 7, 1] = 255
    W_big2 = {k: v.copy() for k, v in W.items()}
    W_big2["down_q"][e, 7, 16:32] = np.uint8(0xA2)  # codes 2 and 10: +1.0, -1.0
    W_big2["down_s"][e, 7, 1] = 254
    uses = (idx == e).any(axis=1)
    assert uses.any()
    for mx in (0, 1, 2):
        y = o.forward(W, x, idx, w, nthreads=1, mx=mx)
        assert np.isfinite(y).all(), mx
        assert np.array_equal(y, o.forward(W_ref, x, idx, w, nthreads=1, mx=mx)), mx
        yb = o.forward(W_big, x, idx, w, nthreads=1, mx=mx)
        assert np.array_equal(yb, o.forward(W_big2, x, idx, w, nthreads=1, mx=mx)), mx
        assert np.all(np.abs(yb[uses, 7]) > 1e30), mx


# ------------------------------------------------------------- P11 LatentMoE wrapper
def check_rmsnorm(o):
    """RMSNorm by hand on a 3-4 vector and the closed form of a constant vector; with
    eps = 0 scaling the input by a power of two leaves the output bit-identical."""
    r = o.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0], np.float32), 0.0)
    rms = math.sqrt(12.5)
    assert abs(r[0] - 3 / rms) <= 1e-15 and abs(r[1] - 8 / rms) <= 1e-15
    c, eps, n = 0.25, 1e-3, 64
    r = o.rmsnorm(np.full(n, c), np.full(n, 1.5, np.float32), eps)
    assert np.allclose(r, 1.5 * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    a = np.random.default_rng(61).standard_normal(100)
    g = (1 + 0.1 * np.random.default_rng(62).standard_normal(100)).astype(np.float32)
    assert np.array_equal(o.rmsnorm(a, g, 0.0), o.rmsnorm(a * 2.0 ** 37, g, 0.0))


def _latent_tiny():
    import synth
    lc = synth.LATENT["latent_tiny"]
    cfg = lc.experts
    dense = dict(synth.latent_dense_host(lc))
    W = synth.weights_host(cfg)
    h, logits, bias = synth.latent_activations(lc)
    return lc, cfg, dense, W, h, logits, bias


def _ldense(dense, eps):
    return {"w_dn": dense["w_down"], "w_up": dense["w_up"], "norm": dense["norm"], "eps": eps,
            "sg": dense["shared_gate"], "su": dense["shared_up"], "sd": dense["shared_down"]}


def check_latent_composition(o):
    """The block is its stages in order: x = Wdn h (fsum of exact products), the
    routed aggregate of the oracle's own forward on x rounded once to fp32 (no other
    rounding between the projection and the experts), RMSNorm on that aggregate,
    Wup, plus the shared experts as one SiTU-GLU expert of width Fs."""
    lc, cfg, dense, W, h, logits, bias = _latent_tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    out, xl, agg = o.latent_forward(_ldense(dense, lc.eps), W, h, idx, w, nthreads=2, want_parts=True)
    Wdn, Wup = dense["w_down"].astype(np.float64), dense["w_up"].astype(np.float64)
    for t in range(h.shape[0]):
        for i in range(0, cfg.D, 37):
            terms = Wdn[i] * h[t].astype(np.float64)
            assert abs(xl[t, i] - math.fsum(terms)) <= 1e-12 * math.fsum(np.abs(terms)), (t, i)
    y, ytk, _ = o.forward(W, xl.astype(np.float32), idx, w, want_pairs=True)
    want_agg = np.zeros_like(agg)
    for k in range(cfg.K):
        want_agg += w[:, k:k + 1].astype(np.float64) * ytk[:, k]
    assert np.array_equal(agg, want_agg)
    for t in range(h.shape[0]):
        r = o.rmsnorm(agg[t], dense["norm"], lc.eps)
        sh = o.expert(dense["shared_gate"], dense["shared_up"], dense["shared_down"], h[t])["y"]
        for d in range(0, lc.Dh, 29):
            terms = Wup[d] * r
            want = math.fsum(terms) + sh[d]
            assert abs(out[t, d] - want) <= 1e-6 * (math.fsum(np.abs(terms)) + abs(sh[d])) + 1e-30, (t, d)


def check_latent_zero_paths(o):
    """Zero shared down-projection: out is the routed branch alone; zero up-projection:
    out is the shared experts alone (each path can be switched off on its own)."""
    lc, cfg, dense, W, h, logits, bias = _latent_tiny()
    idx, w, _ = o.route(logits, bias, cfg.K)
    d0 = _ldense(dense, lc.eps)
    full = o.latent_forward(d0, W, h, idx, w, nthreads=2)
    no_sh = o.latent_forward(dict(d0, sd=np.zeros_like(d0["sd"])), W, h, idx, w, nthreads=2)
    no_up = o.latent_forward(dict(d0, w_up=np.zeros_like(d0["w_up"])), W, h, idx, w, nthreads=2)
    for t in range(h.shape[0]):
        sh = o.expert(dense["shared_gate"], dense["shared_up"], dense["shared_down"], h[t])["y"]
        assert np.array_equal(no_up[t], sh.astype(np.float32)), t
    assert np.allclose(full, no_sh.astype(np.float64) + no_up, rtol=1e-6, atol=1e-6)
    assert np.abs(no_sh).max() > 0 and np.abs(no_up).max() > 0


ALL_CHECKS = [
    check_decode_closed_form, check_decode_conventions, check_layout_fixture, check_scale_groups,
    check_dequant_matches_codes, check_expert_brute_force, check_route_brute_force,
    check_route_invariants, check_route_bias_reading, check_route_nan, check_situ,
    check_forward_pairs, check_forward_combine, check_chunk_equals_tokens, check_group,
    check_route_topp_definition, check_route_topp_off_and_monotone, check_forward_pruned, check_group_pruned,
    check_e4m3_decode, check_mx_quant_exact_values, check_mx_quant_brute, check_mx_quant_special,
    check_mx_quant_two_parts, check_forward_mx, check_forward_mx_weight_scale_255,
    check_rmsnorm, check_latent_composition, check_latent_zero_paths,
]
# check_gate_moments is run separately (it pins the generator, and is the slowest)
