/*
 * k3moe_oracle.c -- plain, slow CPU oracle for the Kimi K3 "Stable LatentMoE"
 * routed-expert block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The product (the HIP library) never
 * calls it and shares no code, header or table with it.
 *
 * Pages it follows (cited by title and section below):
 *   [PR676] colibri PR #676, "Kimi K3 engine: native-MXFP4 expert streaming, KDA +
 *           gated NoPE MLA + AttnRes + LatentMoE": summary bullets, "It runs the
 *           full model", the chunked-prefill paragraph, "What's in the commits".
 *   [PR684] colibri PR #684, "Kimi K3: integrate coli chat, API, and Web": the
 *           MXFP4-kernel commit message and the engine commit message.
 *   [LC21]  llama.cpp fork PR #21, "Adding kimi-k3 arch test and saver fix": the
 *           kimi-k3 arch commit and the PR description.
 *
 * Precision: decoded weights are fp32 (the closed form rounded once to fp32);
 * every sum, the activation and the combine run in double; outputs are cast to
 * fp32 once at the end.  The router's selection key is an fp32 value (see
 * k3o_route).  Built at -O2 without fast-math and with FP contraction off.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ MXFP4 decode */

/* e2m1 magnitudes, indexed by the code's low three bits (exponent e1 e0, mantissa m).
 * The pages name e2m1 but do not print the table ([PR676] summary: 4-bit e2m1 codes
 * with one ue8m0 scale per 32 inputs; [LC21] arch commit: the code assignment is
 * the one ggml's MXFP4 uses; [PR684] int8 commit: twice every e2m1 value is an
 * exact int8).  This is the standard OCP e2m1 value set. */
static const double E2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* One weight from a 4-bit code and its group's scale byte:
 * w = v * 2^(s - 127), v = (-1)^bit3 * E2M1[code & 7]   ([PR684] MXFP4 commit: the
 * code's bit 3 is the sign, the scale byte is a biased power-of-two exponent).
 * The product is exact in double; it is then rounded once to fp32.  Every value
 * below 2^128 has at most two significant bits and magnitude >= 2^-128, so it is
 * representable in fp32 (subnormals included); anything >= 2^128 overflows to a
 * signed infinity, as IEEE 754 rounding to nearest prescribes.  Code 8 is -0.0. */
float k3o_decode(unsigned code, unsigned scale)
{
    double v = E2M1[code & 7u];
    if (code & 8u) v = -v;
    double w = v * ldexp(1.0, (int)(scale & 0xFFu) - 127);
    if (fabs(w) >= 0x1p128) return (float)copysign(INFINITY, w);
    return (float)w;
}

/* Fill a 16 x 256 table: table[code * 256 + s] = k3o_decode(code, s). */
void k3o_decode_table(float *table)
{
    for (unsigned c = 0; c < 16; ++c)
        for (unsigned s = 0; s < 256; ++s) table[c * 256 + s] = k3o_decode(c, s);
}

/* Dequantize one MXFP4 matrix.  Packed q is [O, I/2] bytes, the LOW nibble holding
 * the even column and the high nibble the odd column; scales s are [O, I/32], one
 * per 32 consecutive inputs of a row ([PR684] MXFP4 commit).  out is [O, I] fp32. */
void k3o_dequant(const uint8_t *q, const uint8_t *s, int64_t O, int64_t I, float *out)
{
    float table[16 * 256]; /* every (code, scale) pair, each entry from k3o_decode */
    k3o_decode_table(table);
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t i = 0; i < I; ++i) {
            uint8_t byte = q[o * (I / 2) + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
            unsigned scale = s[o * (I / 32) + i / 32];
            out[o * I + i] = table[code * 256 + scale];
        }
    }
}

/* ------------------------------------------------------------------------ router */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

typedef struct { float key; int32_t id; } cand_t;

/* Larger key first; equal keys -> lower expert id first. */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

/* Sigmoid router with a score-correction bias, top-K, renormalized on raw scores
 * ([PR684] engine commit, Stable LatentMoE bullet; [PR676] summary: 896 experts
 * per layer, top-16).
 *   score_e = sigma(l_e)                         (double)
 *   key_e   = fl32( fl32(score_e) + bias_e )     (the bias only steers selection)
 *   select the K largest keys, ties to the lower id, in descending key order
 *   w_k     = score_{e_k} / sum_j score_{e_j}    (double, cast to fp32)
 * A NaN key counts as -inf.  gap[t] = key_(K) - key_(K+1) (inf when K == E) is
 * the selection's margin, reported so near-ties can be counted.
 * logits [T, E], bias [E]; idx [T, K] int32, w [T, K] fp32, gap [T] (nullable). */
/* Scores and the top-K candidates (descending key, ties to the lower id) of one
 * token; c[0..K-1] is the selection in slot order. */
static void select_token(const float *l, const float *bias, int32_t E, cand_t *c, double *score)
{
    for (int32_t e = 0; e < E; ++e) {
        score[e] = sigmoid((double)l[e]);
        float s32 = (float)score[e];
        float key = s32 + bias[e];
        if (isnan(key)) key = -INFINITY;
        c[e].key = key;
        c[e].id = e;
    }
    qsort(c, (size_t)E, sizeof(cand_t), cand_cmp);
}

void k3o_route(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K,
               int32_t *idx, float *w, double *gap)
{
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)E);
    double *score = (double *)malloc(sizeof(double) * (size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        select_token(logits + (int64_t)t * E, bias, E, c, score);
        double denom = 0.0;
        for (int32_t k = 0; k < K; ++k) denom += score[c[k].id];
        for (int32_t k = 0; k < K; ++k) {
            idx[(int64_t)t * K + k] = c[k].id;
            w[(int64_t)t * K + k] = (float)(score[c[k].id] / denom);
        }
        if (gap) gap[t] = (K < E) ? (double)c[K - 1].key - (double)c[K].key : INFINITY;
    }
    free(c);
    free(score);
}

/* The router followed by top-p pruning ([PR676] K3_TOPP paragraph; [PR684] engine
 * commit, K3_TOPP bullet): of the K selected experts, keep those with the largest
 * routing weights until their cumulative weight reaches p, drop the low-weight
 * tail, and renormalize the kept raw scores.  Readings of the rule:
 *   - weight order: descending raw score sigma (equal scores: lower slot first);
 *   - kept count m: the smallest m whose running sum of scores in that order
 *     reaches p * S, S = sum of the K scores in slot order (double; the running
 *     sum adds in weight order); so the expert that crosses p is kept, and m >= 1;
 *   - p <= 0 or p >= 1 turns pruning off (m = K): the result equals k3o_route;
 *   - output: the kept experts in their original slot order in slots 0..m-1,
 *     w = score / (sum of kept scores in slot order); slots m..K-1 hold id -1
 *     (pruned) and weight 0.
 * n_kept [T] (nullable) receives m; gap as in k3o_route. */
void k3o_route_topp(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K, double p,
                    int32_t *idx, float *w, int32_t *n_kept, double *gap)
{
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)E);
    double *score = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    int *kept = (int *)malloc(sizeof(int) * (size_t)K);
    for (int32_t t = 0; t < T; ++t) {
        select_token(logits + (int64_t)t * E, bias, E, c, score);
        double S = 0.0;
        for (int32_t k = 0; k < K; ++k) S += score[c[k].id];
        int32_t m = K;
        if (p > 0.0 && p < 1.0) {
            /* slots in weight order: insertion sort, stable, larger score first */
            for (int32_t k = 0; k < K; ++k) {
                int32_t j = k;
                while (j > 0 && score[c[order[j - 1]].id] < score[c[k].id]) {
                    order[j] = order[j - 1];
                    --j;
                }
                order[j] = k;
            }
            const double thr = p * S;
            double cum = 0.0;
            for (m = 0; m < K;) {
                cum += score[c[order[m]].id];
                ++m;
                if (cum >= thr) break;
            }
        }
        for (int32_t k = 0; k < K; ++k) kept[k] = (m == K);
        if (m < K)
            for (int32_t r = 0; r < m; ++r) kept[order[r]] = 1;
        double Sk = 0.0;
        for (int32_t k = 0; k < K; ++k)
            if (kept[k]) Sk += score[c[k].id];
        int32_t j = 0;
        for (int32_t k = 0; k < K; ++k) {
            if (!kept[k]) continue;
            idx[(int64_t)t * K + j] = c[k].id;
            w[(int64_t)t * K + j] = (float)(score[c[k].id] / Sk);
            ++j;
        }
        for (; j < K; ++j) {
            idx[(int64_t)t * K + j] = -1;
            w[(int64_t)t * K + j] = 0.0f;
        }
        if (n_kept) n_kept[t] = m;
        if (gap) gap[t] = (K < E) ? (double)c[K - 1].key - (double)c[K].key : INFINITY;
    }
    free(c);
    free(score);
    free(order);
    free(kept);
}

/* -------------------------------------------------------------------- activation */

/* Generic-beta SiTU-GLU: bg*tanh(g/bg) * sigma(g) * bu*tanh(u/bu).  sigma acts on
 * the gate branch only. */
double k3o_situ_beta(double g, double u, double bg, double bu)
{
    return bg * tanh(g / bg) * sigmoid(g) * bu * tanh(u / bu);
}

/* SiTU-GLU with K3's betas 4 and 25: 4*tanh(g/4)*sigma(g)*25*tanh(u/25)
 * ([PR676] summary, Stable LatentMoE bullet; [PR684] engine commit; [LC21] PR
 * description: situ at betas 4.0 / 25.0).  exp(+large) = inf gives sigma = 0, so
 * the expression saturates without inf/inf; NaN propagates. */
double k3o_situ(double g, double u) { return k3o_situ_beta(g, u, 4.0, 25.0); }

/* ------------------------------------------------------------------- expert FFN */

static void expert_gateup(const float *Wg, const float *Wu, int32_t D, int32_t F, const double *x,
                          double *g, double *u, double *h)
{
    for (int32_t f = 0; f < F; ++f) {
        double ag = 0.0, au = 0.0;
        for (int32_t i = 0; i < D; ++i) {
            ag += (double)Wg[(int64_t)f * D + i] * x[i];
            au += (double)Wu[(int64_t)f * D + i] * x[i];
        }
        if (g) g[f] = ag;
        if (u) u[f] = au;
        h[f] = k3o_situ(ag, au);
    }
}

static void expert_down(const float *Wd, int32_t D, int32_t F, const double *h, double *y)
{
    for (int32_t d = 0; d < D; ++d) {
        double ay = 0.0;
        for (int32_t f = 0; f < F; ++f) ay += (double)Wd[(int64_t)d * F + f] * h[f];
        y[d] = ay;
    }
}

/* One routed expert on one token, on already-decoded fp32 weights
 * Wg, Wu [F, D] and Wd [D, F]:
 *   g_f = sum_i Wg[f,i] x_i,  u_f = sum_i Wu[f,i] x_i     (double, ascending i)
 *   h_f = SiTU(g_f, u_f)
 *   y_d = sum_f Wd[d,f] h_f                                (double, ascending f)
 * ([PR684] engine commit: gate/up, SiTU-GLU, down in the 3584-dim latent space.)
 * Any output pointer may be NULL except y. */
void k3o_expert(const float *Wg, const float *Wu, const float *Wd, int32_t D, int32_t F,
                const float *x, double *g, double *u, double *h, double *y)
{
    double *hh = (double *)malloc(sizeof(double) * (size_t)F);
    double *xd = (double *)calloc((size_t)D, sizeof(double));
    for (int32_t i = 0; i < D; ++i) xd[i] = x[i];
    expert_gateup(Wg, Wu, D, F, xd, g, u, hh);
    free(xd);
    if (h)
        for (int32_t f = 0; f < F; ++f) h[f] = hh[f];
    expert_down(Wd, D, F, hh, y);
    free(hh);
}

/* ---------------------------------------------------- MXFP8 activations (variant) */

/* The low-precision-activation variant of the chunk path: the GPU analog of the
 * pages' per-32 int8 activations ([PR684] int8-activation commit, K3_IDOT: the
 * activations are quantized in groups of 32 and multiplied with the MXFP4
 * weights as they are).  Here the groups are OCP MX: 32 consecutive values share
 * one E8M0 scale 2^(s-127) and each value is an FP8 E4M3 code (bias 7, three
 * mantissa bits, subnormals, largest finite 448, 0x7F/0xFF NaN).  For a group:
 *   amax = max |v|;  amax = 0: s = 0 and every code 0;
 *   otherwise s = clamp(floor(log2 amax) - 8 + 127, 0, 254) (8 = E4M3's largest
 *   exponent), y = v / 2^(s-127), clamped to [-448, 448], rounded to the nearest
 *   E4M3 value with ties to the even code;
 *   a group holding a NaN or an infinity gets the E8M0 NaN scale s = 255 and
 *   NaN codes 0x7F.
 * Every step is exact in double (power-of-two scaling, one rounding). */
double k3o_e4m3_decode(unsigned code)
{
    const unsigned e = (code >> 3) & 15u, m = code & 7u;
    if ((code & 0x7Fu) == 0x7Fu) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, (int)e - 7);
    return (code & 0x80u) ? -mag : mag;
}

static unsigned e4m3_encode(double y) /* |y| <= 448, finite */
{
    const unsigned sign = (y < 0.0 || (y == 0.0 && signbit(y))) ? 0x80u : 0u;
    const double a = fabs(y);
    if (a < ldexp(1.0, -6)) {          /* subnormal range: quantum 2^-9 */
        const double q = nearbyint(ldexp(a, 9));   /* ties to even (default mode) */
        return sign | (unsigned)q;     /* q = 8 is the smallest normal, code 0x08 */
    }
    int e2;
    (void)frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                    /* floor(log2 a), in [-6, 8] */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {
        m = 0.0;
        ++e;
    }
    unsigned code = (unsigned)((e + 7) << 3) | (unsigned)m;
    if (code > 0x7Eu) code = 0x7Eu;    /* saturate at 448 */
    return sign | code;
}

void k3o_mx_quant(const float *v, int64_t n, uint8_t *codes, uint8_t *scales)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        const float *g = v + 32 * b;
        double amax = 0.0;
        int finite = 1;
        for (int i = 0; i < 32; ++i) {
            if (!isfinite(g[i])) finite = 0;
            else if (fabs((double)g[i]) > amax) amax = fabs((double)g[i]);
        }
        if (!finite) {
            scales[b] = 255;
            for (int i = 0; i < 32; ++i) codes[32 * b + i] = 0x7F;
            continue;
        }
        if (amax == 0.0) {
            scales[b] = 0;
            for (int i = 0; i < 32; ++i) codes[32 * b + i] = (uint8_t)(signbit(g[i]) ? 0x80 : 0);
            continue;
        }
        int e2;
        (void)frexp(amax, &e2);
        int s = (e2 - 1) - 8 + 127;
        if (s < 0) s = 0;
        if (s > 254) s = 254;
        scales[b] = (uint8_t)s;
        for (int i = 0; i < 32; ++i) {
            double y = ldexp((double)g[i], 127 - s);
            if (y > 448.0) y = 448.0;
            if (y < -448.0) y = -448.0;
            codes[32 * b + i] = (uint8_t)e4m3_encode(y);
        }
    }
}

/* Value of one MXFP8 element (scale byte 255 is the E8M0 NaN).  Every value of a
 * block quantized from finite fp32 input is an fp32 value: its scale exponent
 * lies in [-127, 119] and E4M3 carries four significant bits. */
static float mx_value(uint8_t code, uint8_t scale)
{
    return scale == 255 ? NAN : (float)(k3o_e4m3_decode(code) * ldexp(1.0, (int)scale - 127));
}

/* Quantization in `parts` MXFP8 parts (1 or 2): part 0 is v quantized as above;
 * part 1 is the fp32 residual v - part0 quantized the same way (the residual is
 * exact in fp32: part 0 is v rounded to nearest on a grid coarser than v's, so
 * it lies within a factor two of v or is zero).  codes [parts][n],
 * scales [parts][n/32]. */
void k3o_mx_quant_parts(const float *v, int64_t n, int32_t parts, uint8_t *codes, uint8_t *scales)
{
    k3o_mx_quant(v, n, codes, scales);
    if (parts < 2) return;
    float *r = (float *)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) r[i] = v[i] - mx_value(codes[i], scales[i / 32]);
    k3o_mx_quant(r, n, codes + n, scales + n / 32);
    free(r);
}

/* v -> MXFP8 in `parts` parts -> the sum of the parts' values, in double. */
static void mx_roundtrip(const float *v, int64_t n, int32_t parts, double *out)
{
    uint8_t *c = (uint8_t *)malloc((size_t)(2 * n)), *sc = (uint8_t *)malloc((size_t)(2 * (n / 32)));
    k3o_mx_quant_parts(v, n, parts, c, sc);
    for (int64_t i = 0; i < n; ++i) {
        out[i] = mx_value(c[i], sc[i / 32]);
        if (parts > 1) out[i] += mx_value(c[n + i], sc[n / 32 + i / 32]);
    }
    free(c);
    free(sc);
}

/* k3o_expert with MXFP8 activations in `parts` parts: x is quantized as above,
 * g and u are sums over the quantized x, h = SiTU(g, u) is rounded to fp32 and
 * quantized the same way (in groups of 32 consecutive f), and y is the sum over
 * that h; sums in double, ascending index. */
void k3o_expert_mx(const float *Wg, const float *Wu, const float *Wd, int32_t D, int32_t F,
                   int32_t parts, const float *x, double *h, double *y)
{
    double *xq = (double *)malloc(sizeof(double) * (size_t)D);
    float *hf = (float *)malloc(sizeof(float) * (size_t)F);
    double *hd = (double *)malloc(sizeof(double) * (size_t)F);
    mx_roundtrip(x, D, parts, xq);
    expert_gateup(Wg, Wu, D, F, xq, NULL, NULL, hd);
    for (int32_t f = 0; f < F; ++f) hf[f] = (float)hd[f];
    mx_roundtrip(hf, F, parts, hd);
    if (h)
        for (int32_t f = 0; f < F; ++f) h[f] = hd[f];
    expert_down(Wd, D, F, hd, y);
    free(xq);
    free(hf);
    free(hd);
}

/* ----------------------------------------------------------------- block forward */

/* Progress of k3o_forward: every n-th expert finished is reported on stderr (n = 0:
 * silent), so a long run shows that it advances. */
static int32_t g_progress = 0;
void k3o_set_progress(int32_t every) { g_progress = every; }

/* The routed-expert block for T tokens given their routing (idx [T,K], w [T,K]):
 *   y_t = sum_{k=0}^{K-1} w_{t,k} * expert_{idx[t,k]}(x_t)     (double, k order)
 * A slot holding id -1 was pruned (k3o_route_topp) and contributes nothing.
 * Weights: gq/uq [E, F, D/2], gs/us [E, F, D/32], dq [E, D, F/2], ds [E, D, F/32].
 * Each token is computed exactly as it would be alone; the loop visits the union
 * of routed experts and decodes each of them once (the pages' chunk loads each
 * unique expert once, [PR676] chunked-prefill paragraph), which does not change
 * any pair's arithmetic.  ytk (nullable) receives the per-pair expert outputs
 * [T, K, D] in double; hk (nullable) the per-pair activations [T, K, F].
 * Returns 0, or -1 if an index is out of range or memory runs out. */
static int forward_impl(int32_t E, int32_t D, int32_t F,
                        const uint8_t *gq, const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                        const uint8_t *dq, const uint8_t *ds,
                        const float *x, int32_t T, const int32_t *idx, const float *w, int32_t K,
                        float *y, double *ytk, double *hk, int32_t nthreads, int32_t mx_parts)
{
    int64_t P = (int64_t)T * K;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] != -1 && (idx[p] < 0 || idx[p] >= E)) return -1;

    double *yp = ytk ? ytk : (double *)malloc(sizeof(double) * (size_t)(P * D));
    if (!yp) return -1;

    /* union of routed experts, ascending */
    int32_t *used = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t nu = 0;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] >= 0) used[idx[p]] = 1;
    for (int32_t e = 0; e < E; ++e)
        if (used[e]) list[nu++] = e;

    const int64_t gq_n = (int64_t)F * D / 2, gs_n = (int64_t)F * D / 32;
    const int64_t dq_n = (int64_t)D * F / 2, ds_n = (int64_t)D * F / 32;
    int failed = 0;
    int32_t done = 0;

#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        float *Wg = (float *)malloc(sizeof(float) * (size_t)F * D);
        float *Wu = (float *)malloc(sizeof(float) * (size_t)F * D);
        float *Wd = (float *)malloc(sizeof(float) * (size_t)D * F);
#pragma omp for schedule(dynamic, 1)
        for (int32_t j = 0; j < nu; ++j) {
            if (!Wg || !Wu || !Wd) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            int32_t e = list[j];
            k3o_dequant(gq + e * gq_n, gs + e * gs_n, F, D, Wg);
            k3o_dequant(uq + e * gq_n, us + e * gs_n, F, D, Wu);
            k3o_dequant(dq + e * dq_n, ds + e * ds_n, D, F, Wd);
            for (int64_t p = 0; p < P; ++p) {
                if (idx[p] != e) continue;
                int64_t t = p / K;
                if (mx_parts)
                    k3o_expert_mx(Wg, Wu, Wd, D, F, mx_parts, x + t * D, hk ? hk + p * F : NULL, yp + p * D);
                else
                    k3o_expert(Wg, Wu, Wd, D, F, x + t * D, NULL, NULL,
                               hk ? hk + p * F : NULL, yp + p * D);
            }
            if (g_progress > 0) {
                int32_t n;
#pragma omp atomic capture
                n = ++done;
                if (n % g_progress == 0 || n == nu) {
                    fprintf(stderr, "[oracle] %d / %d experts\n", n, nu);
                    fflush(stderr);
                }
            }
        }
        free(Wg);
        free(Wu);
        free(Wd);
    }

    if (!failed) {
        for (int32_t t = 0; t < T; ++t)
            for (int32_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int32_t k = 0; k < K; ++k)
                    if (idx[(int64_t)t * K + k] >= 0)
                        acc += (double)w[(int64_t)t * K + k] * yp[((int64_t)t * K + k) * D + d];
                y[(int64_t)t * D + d] = (float)acc;
            }
    }
    free(used);
    free(list);
    if (!ytk) free(yp);
    return failed ? -1 : 0;
}

int k3o_forward(int32_t E, int32_t D, int32_t F,
                const uint8_t *gq, const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                const uint8_t *dq, const uint8_t *ds,
                const float *x, int32_t T, const int32_t *idx, const float *w, int32_t K,
                float *y, double *ytk, double *hk, int32_t nthreads)
{
    return forward_impl(E, D, F, gq, gs, uq, us, dq, ds, x, T, idx, w, K, y, ytk, hk, nthreads, 0);
}

/* k3o_forward with MXFP8 activations in `parts` (1 or 2) parts (k3o_expert_mx for
 * every pair); the weights are the same closed-form values as in k3o_forward for
 * every scale byte, 255 included ([PR684] MXFP4-kernel commit: w = v * 2^(s-127),
 * and the engine's kernels agree on the s = 0 and s = 255 edge cases); hk receives
 * the dequantized h. */
int k3o_forward_mx(int32_t E, int32_t D, int32_t F,
                   const uint8_t *gq, const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                   const uint8_t *dq, const uint8_t *ds,
                   const float *x, int32_t T, const int32_t *idx, const float *w, int32_t K,
                   float *y, double *ytk, double *hk, int32_t nthreads, int32_t parts)
{
    if (parts < 1 || parts > 2) return -1;
    return forward_impl(E, D, F, gq, gs, uq, us, dq, ds, x, T, idx, w, K, y, ytk, hk, nthreads, parts);
}

/* ------------------------------------------------------------------ chunk grouping */

/* Group a chunk's (token, slot) pairs by expert with a counting sort ([PR676]
 * chunked-prefill paragraph: the MoE loads each unique expert of the chunk once;
 * [PR684] chunked-prefill commit: position lists via counting sort).
 *   counts[e]   number of pairs routed to e (pruned slots, id -1, are skipped)
 *   offsets[e]  exclusive prefix sum of counts (offsets[E] = pairs placed)
 *   perm[...]   pair ids p = t*K + k, grouped by ascending expert and, within an
 *               expert, in ascending p (a counting sort is stable)
 *   uniq[...]   the experts with counts > 0, ascending; *n_unique their number
 * Returns 0, or -1 if an index is out of range. */
int k3o_group(const int32_t *idx, int32_t T, int32_t K, int32_t E, int32_t *counts,
              int32_t *offsets, int32_t *perm, int32_t *uniq, int32_t *n_unique)
{
    int64_t P = (int64_t)T * K;
    memset(counts, 0, sizeof(int32_t) * (size_t)E);
    for (int64_t p = 0; p < P; ++p) {
        if (idx[p] == -1) continue;
        if (idx[p] < 0 || idx[p] >= E) return -1;
        counts[idx[p]]++;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = idx[p];
        if (e == -1) continue;
        perm[offsets[e] + fill[e]] = (int32_t)p;
        fill[e]++;
    }
    free(fill);
    int32_t nu = 0;
    for (int32_t e = 0; e < E; ++e)
        if (counts[e] > 0) uniq[nu++] = e;
    *n_unique = nu;
    return 0;
}

/* -------------------------------------------------------------- LatentMoE wrapper */

/* RMSNorm of n values: r_i = g_i * a_i / sqrt(mean(a^2) + eps), in double.
 * Returns the root mean square sqrt(mean(a^2) + eps). */
double k3o_rmsnorm(const double *a, int32_t n, const float *g, double eps, double *r)
{
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += a[i] * a[i];
    const double rms = sqrt(ss / n + eps);
    for (int32_t i = 0; i < n; ++i) r[i] = (double)g[i] * (a[i] / rms);
    return rms;
}

/* y[o] = sum_i W[o, i] x[i] for W [O, I] (float values), x double; ascending i. */
static void dense(const float *W, int32_t O, int32_t I, const double *x, double *y)
{
    for (int32_t o = 0; o < O; ++o) {
        double acc = 0.0;
        for (int32_t i = 0; i < I; ++i) acc += (double)W[(int64_t)o * I + i] * x[i];
        y[o] = acc;
    }
}

/* The block around the routed experts ([PR684] engine commit, Stable LatentMoE
 * bullet: latent 7168 <-> 3584 projections around the experts, RMSNorm on the
 * aggregate, two fused shared experts, SiTU-GLU; [PR676] summary: the routed
 * experts run in a 3584-dim latent space behind shared down/up projections,
 * plus two fused full-width shared experts).  The pages give no formulas; the
 * plainest reading, per token with hidden state h [Dh]:
 *   x   = fp32(Wdn h)                     latent input of the routed experts: the
 *                                         projection rounded once to fp32 (the
 *                                         engine's activations are fp32; the pages
 *                                         round nothing between the projection
 *                                         and the experts)
 *   a   = sum_k w_k E_k(x)                the routed aggregate (k3o_forward)
 *   r   = RMSNorm(a) with weight gn, eps  "on the aggregate": in the latent space
 *   y   = Wup r                           back to the full width
 *   s   = Sd SiTU(Sg h, Su h)             the two shared experts fused into one
 *                                         SiTU-GLU MLP of width Fs (both halves)
 *   out = y + s
 * Dense weights: Wdn [Dl, Dh], Wup [Dh, Dl], Sg/Su [Fs, Dh], Sd [Dh, Fs] as float
 * (their bf16 values), gn [Dl]; expert weights and routing as in k3o_forward on
 * the latent x.  Sums in double; out [T, Dh] fp32; xl (nullable) receives Wdn h
 * [T, Dl] before the fp32 rounding and agg (nullable) a [T, Dl], in double.  Returns 0, or -1 as
 * k3o_forward does. */
int k3o_latent_forward(int32_t Dh, int32_t Dl, int32_t Fs,
                       const float *Wdn, const float *Wup, const float *gn, double eps,
                       const float *Sg, const float *Su, const float *Sd,
                       int32_t E, int32_t F,
                       const uint8_t *gq, const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                       const uint8_t *dq, const uint8_t *ds,
                       const float *h, int32_t T, const int32_t *idx, const float *w, int32_t K,
                       float *out, double *xl, double *agg, int32_t nthreads)
{
    float *x32 = (float *)malloc(sizeof(float) * (size_t)T * Dl);
    float *y32 = (float *)malloc(sizeof(float) * (size_t)T * Dl);
    double *ytk = (double *)malloc(sizeof(double) * (size_t)T * K * Dl);
    if (!x32 || !y32 || !ytk) {
        free(x32);
        free(y32);
        free(ytk);
        return -1;
    }
#pragma omp parallel for num_threads(nthreads > 0 ? nthreads : 1) schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        double *hd = (double *)malloc(sizeof(double) * (size_t)Dh);
        double *xd = (double *)malloc(sizeof(double) * (size_t)Dl);
        for (int32_t i = 0; i < Dh; ++i) hd[i] = h[(int64_t)t * Dh + i];
        dense(Wdn, Dl, Dh, hd, xd);
        for (int32_t i = 0; i < Dl; ++i) {
            x32[(int64_t)t * Dl + i] = (float)xd[i];
            if (xl) xl[(int64_t)t * Dl + i] = xd[i];
        }
        free(hd);
        free(xd);
    }
    int rc = k3o_forward(E, Dl, F, gq, gs, uq, us, dq, ds, x32, T, idx, w, K, y32, ytk, NULL, nthreads);
    if (rc == 0) {
#pragma omp parallel for num_threads(nthreads > 0 ? nthreads : 1) schedule(dynamic, 1)
        for (int32_t t = 0; t < T; ++t) {
            double *a = (double *)malloc(sizeof(double) * (size_t)Dl);
            double *r = (double *)malloc(sizeof(double) * (size_t)Dl);
            double *y = (double *)malloc(sizeof(double) * (size_t)Dh);
            double *s = (double *)malloc(sizeof(double) * (size_t)Dh);
            for (int32_t i = 0; i < Dl; ++i) {
                double acc = 0.0;
                for (int32_t k = 0; k < K; ++k)
                    if (idx[(int64_t)t * K + k] >= 0)
                        acc += (double)w[(int64_t)t * K + k] * ytk[((int64_t)t * K + k) * Dl + i];
                a[i] = acc;
                if (agg) agg[(int64_t)t * Dl + i] = acc;
            }
            k3o_rmsnorm(a, Dl, gn, eps, r);
            dense(Wup, Dh, Dl, r, y);
            k3o_expert(Sg, Su, Sd, Dh, Fs, h + (int64_t)t * Dh, NULL, NULL, NULL, s);
            for (int32_t i = 0; i < Dh; ++i) out[(int64_t)t * Dh + i] = (float)(y[i] + s[i]);
            free(a);
            free(r);
            free(y);
            free(s);
        }
    }
    free(x32);
    free(y32);
    free(ytk);
    return rc;
}
