"""The pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/k3moe_oracle.c``, plants ONE mistake by a textual
replacement, builds the copy with gcc into a temporary directory and runs every
pin against it.  At least one pin must fail.  Everything here runs on the CPU.
"""
import os
import shutil
import tempfile

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "k3moe_oracle.c")

MUTANTS = [
    ("nibble order swapped",
     "(i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)", "(i % 2 == 0) ? (byte >> 4) : (byte & 0x0Fu)"),
    ("sign bit ignored", "if (code & 8u) v = -v;", ""),
    ("scale bias 128", "(int)(scale & 0xFFu) - 127", "(int)(scale & 0xFFu) - 128"),
    ("e2m1 table entry", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}"),
    ("s=255 read as NaN", "if (fabs(w) >= 0x1p128)", "if ((scale & 0xFFu) == 255u) return NAN;\n    if (fabs(w) >= 0x1p128)"),
    ("subnormals flushed", "    return (float)w;\n}", "    return (fabs(w) < 0x1p-126) ? (float)copysign(0.0, w) : (float)w;\n}"),
    ("wrong scale group", "s[o * (I / 32) + i / 32]", "s[o * (I / 32) + i / 64]"),
    ("bias on logits", "score[e] = sigmoid((double)l[e]);\n        float s32 = (float)score[e];\n        float key = s32 + bias[e];",
     "score[e] = sigmoid((double)l[e]);\n        float s32 = (float)sigmoid((double)l[e] + bias[e]);\n        float key = s32;"),
    ("weights from biased keys", "denom += score[c[k].id];", "denom += c[k].key;"),
    ("numerator from biased key", "w[(int64_t)t * K + k] = (float)(score[c[k].id] / denom);",
     "w[(int64_t)t * K + k] = (float)(c[k].key / denom);"),
    ("ties to higher id", "return (a->id < b->id) ? -1 : (a->id > b->id);", "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    ("renormalize over all experts", "for (int32_t k = 0; k < K; ++k) denom += score[c[k].id];",
     "for (int32_t k = 0; k < E; ++k) denom += score[c[k].id];"),
    ("NaN not demoted", "if (isnan(key)) key = -INFINITY;", ""),
    ("sigmoid sign", "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    ("betas swapped", "k3o_situ_beta(g, u, 4.0, 25.0)", "k3o_situ_beta(g, u, 25.0, 4.0)"),
    ("sigma on up branch", "sigmoid(g) * bu", "sigmoid(u) * bu"),
    ("gate/up swapped", "h[f] = k3o_situ(ag, au);", "h[f] = k3o_situ(au, ag);"),
    ("down transposed", "Wd[(int64_t)d * F + f]", "Wd[(int64_t)f * D + d]"),
    ("dropped last input term", "for (int32_t i = 0; i < D; ++i) {", "for (int32_t i = 0; i < D - 1; ++i) {"),
    ("wrong token for a pair", "x + t * D, NULL, NULL", "x + (p % T) * D, NULL, NULL"),
    ("combine ignores weights", "acc += (double)w[(int64_t)t * K + k] * yp[", "acc += yp["),
    ("combine drops last slot",
     "for (int32_t k = 0; k < K; ++k)\n                    if (idx[(int64_t)t * K + k] >= 0)\n                        acc += (double)w[(int64_t)t * K + k] * yp[",
     "for (int32_t k = 0; k < K - 1; ++k)\n                    if (idx[(int64_t)t * K + k] >= 0)\n                        acc += (double)w[(int64_t)t * K + k] * yp["),
    ("group order unstable", "for (int64_t p = 0; p < P; ++p) {\n        int32_t e = idx[p];\n        if (e == -1) continue;",
     "for (int64_t p = P - 1; p >= 0; --p) {\n        int32_t e = idx[p];\n        if (e == -1) continue;"),
    ("union misses singletons", "if (counts[e] > 0) uniq[nu++] = e;", "if (counts[e] > 1) uniq[nu++] = e;"),
    ("top-p in slot order", "while (j > 0 && score[c[order[j - 1]].id] < score[c[k].id])", "while (0)"),
    ("top-p drops the crossing expert", "++m;\n                if (cum >= thr) break;", "if (cum >= thr) break;\n                ++m;"),
    ("top-p renormalizes over all K", "if (kept[k]) Sk += score[c[k].id];", "Sk += score[c[k].id];"),
    ("top-p threshold on weights of all experts", "const double thr = p * S;", "const double thr = p * S * 1.05;"),
    ("group keeps pruned pairs", "if (idx[p] == -1) continue;\n        if (idx[p] < 0", "if (idx[p] == -1) { counts[0]++; continue; }\n        if (idx[p] < 0"),
    ("mx scale offset 7", "int s = (e2 - 1) - 8 + 127;", "int s = (e2 - 1) - 7 + 127;"),
    ("mx ties away from zero", "double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);", "double m = round((ldexp(a, -e) - 1.0) * 8.0);"),
    ("mx subnormal boundary", "if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {"),
    ("e4m3 exponent bias 8", "ldexp(1.0 + m / 8.0, (int)e - 7)", "ldexp(1.0 + m / 8.0, (int)e - 8)"),
    ("mx zero block scale", "            scales[b] = 0;\n", "            scales[b] = 127;\n"),
    ("mx h kept in fp32", "    mx_roundtrip(hf, F, parts, hd);", "    for (int32_t f = 0; f < F; ++f) hd[f] = hf[f];"),
    ("mx x kept in fp32", "    mx_roundtrip(x, D, parts, xq);", "    for (int32_t i = 0; i < D; ++i) xq[i] = x[i];"),
    ("mx weights read 255 as NaN", "            k3o_dequant(dq + e * dq_n, ds + e * ds_n, D, F, Wd);\n",
     "            k3o_dequant(dq + e * dq_n, ds + e * ds_n, D, F, Wd);\n            if (mx_parts)\n"
     "                for (int64_t z = 0; z < (int64_t)D * F; ++z)\n"
     "                    if (ds[e * ds_n + z / 32] == 255) Wd[z] = NAN;\n"),
    ("dequant table transposed", "out[o * I + i] = table[code * 256 + scale];", "out[o * I + i] = table[(scale & 15u) * 256 + (scale >> 4) * 16 + code];"),
    ("mx second part dropped", "        if (parts > 1) out[i] += mx_value(", "        if (0) out[i] += mx_value("),
    ("mx residual of the input", "    for (int64_t i = 0; i < n; ++i) r[i] = v[i] - mx_value(codes[i], scales[i / 32]);",
     "    for (int64_t i = 0; i < n; ++i) r[i] = v[i];"),
    ("rmsnorm without the mean", "const double rms = sqrt(ss / n + eps);", "const double rms = sqrt(ss + eps);"),
    ("rmsnorm weight ignored", "r[i] = (double)g[i] * (a[i] / rms);", "r[i] = a[i] / rms;"),
    ("shared experts dropped", "(float)(y[i] + s[i]);", "(float)(y[i]);"),
    ("dense projection transposed", "acc += (double)W[(int64_t)o * I + i] * x[i];", "acc += (double)W[(int64_t)i * O + o] * x[i];"),
    ("aggregate ignores routing weights", "acc += (double)w[(int64_t)t * K + k] * ytk[", "acc += ytk["),
    ("latent x rounded to bf16", "x32[(int64_t)t * Dl + i] = (float)xd[i];",
     "float xf = (float)xd[i];\n            uint32_t xu;\n            memcpy(&xu, &xf, 4);\n"
     "            xu = (xu + 0x7FFFu + ((xu >> 16) & 1u)) & 0xFFFF0000u;\n            memcpy(&xf, &xu, 4);\n"
     "            x32[(int64_t)t * Dl + i] = xf;"),
    ("offsets inclusive", "offsets[e + 1] = offsets[e] + counts[e];", "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
]


@pytest.fixture(scope="module")
def tmpdir_module():
    d = tempfile.mkdtemp(prefix="k3o_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_mutants_are_distinct():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutation site for {name!r} must occur exactly once"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmpdir_module):
    src = open(SRC).read()
    assert src.count(old) == 1
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    csrc = os.path.join(tmpdir_module, f"{tag}.c")
    with open(csrc, "w") as fh:
        fh.write(src.replace(old, new))
    lib = oracle.build(force=True, src=csrc, out=os.path.join(tmpdir_module, f"{tag}.so"))
    mut = oracle.Oracle(lib)
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(mut)
        except (AssertionError, ValueError) as exc:  # ValueError: oracle rejected its own output
            failures.append((check.__name__, str(exc)[:80]))
    assert failures, f"no pin catches the planted mistake {name!r}"
