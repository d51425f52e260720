/* Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU
 * oracle (test infrastructure): every exported function on small inputs,
 * including the edge cases (scale bytes 0 and 255, code 8, NaN and tied logits,
 * pruned slots, zero and non-finite MX blocks), with a few invariants checked.
 * Exit status 0 when every check holds and the sanitizers report nothing. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float k3o_decode(unsigned code, unsigned scale);
void k3o_decode_table(float *table);
void k3o_dequant(const uint8_t *q, const uint8_t *s, int64_t O, int64_t I, float *out);
void k3o_route(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K, int32_t *idx, float *w,
               double *gap);
void k3o_route_topp(const float *logits, const float *bias, int32_t T, int32_t E, int32_t K, double p, int32_t *idx,
                    float *w, int32_t *n_kept, double *gap);
double k3o_situ(double g, double u);
int k3o_forward(int32_t E, int32_t D, int32_t F, const uint8_t *gq, const uint8_t *gs, const uint8_t *uq,
                const uint8_t *us, const uint8_t *dq, const uint8_t *ds, const float *x, int32_t T, const int32_t *idx,
                const float *w, int32_t K, float *y, double *ytk, double *hk, int32_t nthreads);
int k3o_forward_mx(int32_t E, int32_t D, int32_t F, const uint8_t *gq, const uint8_t *gs, const uint8_t *uq,
                   const uint8_t *us, const uint8_t *dq, const uint8_t *ds, const float *x, int32_t T,
                   const int32_t *idx, const float *w, int32_t K, float *y, double *ytk, double *hk, int32_t nthreads,
                   int32_t parts);
void k3o_mx_quant_parts(const float *v, int64_t n, int32_t parts, uint8_t *codes, uint8_t *scales);
double k3o_rmsnorm(const double *a, int32_t n, const float *g, double eps, double *r);
int k3o_latent_forward(int32_t Dh, int32_t Dl, int32_t Fs, const float *Wdn, const float *Wup, const float *gn,
                       double eps, const float *Sg, const float *Su, const float *Sd, int32_t E, int32_t F,
                       const uint8_t *gq, const uint8_t *gs, const uint8_t *uq, const uint8_t *us, const uint8_t *dq,
                       const uint8_t *ds, const float *h, int32_t T, const int32_t *idx, const float *w, int32_t K,
                       float *out, double *xl, double *agg, int32_t nthreads);
int k3o_group(const int32_t *idx, int32_t T, int32_t K, int32_t E, int32_t *counts, int32_t *offsets, int32_t *perm,
              int32_t *uniq, int32_t *n_unique);
void k3o_set_progress(int32_t every);

static int fails = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);      \
            ++fails;                                                           \
        }                                                                      \
    } while (0)

static unsigned rng = 2463534242u;
static unsigned next(void) {
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}
static float gauss(void) {
    double a = (next() + 1.0) / 4294967297.0, b = (next() + 1.0) / 4294967297.0;
    return (float)(sqrt(-2.0 * log(a)) * cos(6.283185307179586 * b));
}
static uint8_t *bytes(size_t n, unsigned lo, unsigned hi) {
    uint8_t *p = malloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(lo + next() % (hi - lo + 1));
    return p;
}
static float *normals(size_t n, float sd) {
    float *p = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = sd * gauss();
    return p;
}

int main(void) {
    /* decode: table, special bytes */
    float table[16 * 256];
    k3o_decode_table(table);
    CHECK(table[1 * 256 + 127] == 0.5f && table[8 * 256 + 127] == 0.0f && signbit(table[8 * 256 + 127]));
    CHECK(isinf(table[7 * 256 + 255]) && table[0 * 256 + 255] == 0.0f && table[1 * 256 + 0] > 0.0f);
    CHECK(k3o_decode(1, 255) == ldexpf(1.0f, 127));

    /* dequant of a ragged-looking small matrix with every scale byte */
    const int O = 8, I = 96;
    uint8_t *q = bytes((size_t)O * I / 2, 0, 255), *s = bytes((size_t)O * I / 32, 0, 255);
    float *W = malloc(sizeof(float) * O * I);
    k3o_dequant(q, s, O, I, W);
    CHECK(W[0] == k3o_decode(q[0] & 15u, s[0]) || (isnan(W[0]) && isnan(k3o_decode(q[0] & 15u, s[0]))));

    /* routing with NaN, ties, top-p */
    const int T = 6, E = 40, K = 8;
    float *lg = normals((size_t)T * E, 1.0f), *bias = normals(E, 0.1f);
    lg[3] = NAN;
    lg[E + 5] = lg[E + 6];
    int32_t idx[6 * 8], kept[6];
    float w[6 * 8];
    double gap[6];
    k3o_route(lg, bias, T, E, K, idx, w, gap);
    for (int t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int k = 0; k < K; ++k) sum += w[t * K + k];
        CHECK(fabs(sum - 1.0) < 1e-5 && gap[t] >= 0.0);
    }
    k3o_route_topp(lg, bias, T, E, K, 0.6, idx, w, kept, gap);
    for (int t = 0; t < T; ++t) CHECK(kept[t] >= 1 && kept[t] <= K && (kept[t] == K || idx[t * K + K - 1] == -1));
    CHECK(k3o_situ(0.0, 3.0) == 0.0 && isnan(k3o_situ(NAN, 1.0)));

    /* forward, MX forward, grouping on a small layer; edge scale bytes in expert 1 */
    const int Ef = 6, D = 64, F = 64, Tf = 9, Kf = 2;
    const size_t qn = (size_t)F * D / 2, sn = (size_t)F * D / 32;
    uint8_t *gq = bytes(Ef * qn, 0, 255), *uq = bytes(Ef * qn, 0, 255), *dq = bytes(Ef * qn, 0, 255);
    uint8_t *gs = bytes(Ef * sn, 120, 130), *us = bytes(Ef * sn, 120, 130), *ds = bytes(Ef * sn, 120, 130);
    for (size_t i = 0; i < sn; i += 5) gs[sn + i] = (uint8_t)(i % 2 ? 0 : 255);
    float *x = normals((size_t)Tf * D, 1.0f), *y = malloc(sizeof(float) * Tf * D);
    int32_t fi[9 * 2];
    float fw[9 * 2];
    for (int t = 0; t < Tf; ++t) {
        fi[t * Kf] = t % Ef;
        fi[t * Kf + 1] = (t % 4 == 3) ? -1 : (t + 1) % Ef;
        fw[t * Kf] = 0.75f;
        fw[t * Kf + 1] = 0.25f;
    }
    double *ytk = malloc(sizeof(double) * Tf * Kf * D), *hk = malloc(sizeof(double) * Tf * Kf * F);
    k3o_set_progress(2);
    CHECK(k3o_forward(Ef, D, F, gq, gs, uq, us, dq, ds, x, Tf, fi, fw, Kf, y, ytk, hk, 2) == 0);
    k3o_set_progress(0);
    CHECK(k3o_forward(Ef, D, F, gq, gs, uq, us, dq, ds, x, Tf, fi, fw, Kf, y, NULL, NULL, 1) == 0);
    for (int parts = 1; parts <= 2; ++parts)
        CHECK(k3o_forward_mx(Ef, D, F, gq, gs, uq, us, dq, ds, x, Tf, fi, fw, Kf, y, ytk, hk, 2, parts) == 0);
    CHECK(k3o_forward_mx(Ef, D, F, gq, gs, uq, us, dq, ds, x, Tf, fi, fw, Kf, y, NULL, NULL, 1, 3) == -1);
    fi[0] = Ef + 2;
    CHECK(k3o_forward(Ef, D, F, gq, gs, uq, us, dq, ds, x, Tf, fi, fw, Kf, y, NULL, NULL, 1) == -1);
    fi[0] = 0;
    int32_t counts[6], offsets[7], perm[18], uniq[6], nu = 0;
    CHECK(k3o_group(fi, Tf, Kf, Ef, counts, offsets, perm, uniq, &nu) == 0 && nu == Ef);
    CHECK(offsets[Ef] == Tf * Kf - 2);

    /* MX quantization: ordinary, zero, subnormal, non-finite blocks */
    float v[32 * 4];
    for (int i = 0; i < 32; ++i) {
        v[i] = gauss();
        v[32 + i] = 0.0f;
        v[64 + i] = 1e-40f * (float)(i + 1);
        v[96 + i] = (i == 7) ? INFINITY : gauss();
    }
    uint8_t codes[2 * 128], scales[2 * 4];
    k3o_mx_quant_parts(v, 128, 2, codes, scales);
    CHECK(scales[1] == 0 && scales[3] == 255);

    /* RMSNorm and the LatentMoE block (tiny) */
    double a[5] = {1, -2, 3, 0, 0.5}, r[5];
    float g5[5] = {1, 1, 1, 1, 1};
    CHECK(k3o_rmsnorm(a, 5, g5, 1e-6, r) > 0.0);
    const int Dh = 96, Fs = 64;
    float *Wdn = normals((size_t)D * Dh, 0.1f), *Wup = normals((size_t)Dh * D, 0.1f), *gn = normals(D, 0.1f);
    float *Sg = normals((size_t)Fs * Dh, 0.1f), *Su = normals((size_t)Fs * Dh, 0.1f), *Sd = normals((size_t)Dh * Fs, 0.1f);
    float *h = normals((size_t)Tf * Dh, 1.0f), *out = malloc(sizeof(float) * Tf * Dh);
    double *xl = malloc(sizeof(double) * Tf * D), *agg = malloc(sizeof(double) * Tf * D);
    CHECK(k3o_latent_forward(Dh, D, Fs, Wdn, Wup, gn, 1e-6, Sg, Su, Sd, Ef, F, gq, gs, uq, us, dq, ds, h, Tf, fi, fw,
                             Kf, out, xl, agg, 2) == 0);

    free(q); free(s); free(W); free(lg); free(bias); free(gq); free(uq); free(dq); free(gs); free(us); free(ds);
    free(x); free(y); free(ytk); free(hk); free(Wdn); free(Wup); free(gn); free(Sg); free(Su); free(Sd);
    free(h); free(out); free(xl); free(agg);
    if (fails) fprintf(stderr, "%d checks failed\n", fails);
    else printf("oracle driver: all checks passed\n");
    return fails ? 1 : 0;
}
