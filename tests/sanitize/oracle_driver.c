/*
 * oracle_driver.c -- runs every oracle entry point on small seeded inputs,
 * edge cases included, so that a host AddressSanitizer / UndefinedBehavior-
 * Sanitizer build of the oracle sees each of its loops and allocations.
 * Test infrastructure only; it checks no values (the pins do that).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_round(const double *x, double *y, int64_t n, int dtype);
void orc_project(const double *K, const double *W, int64_t rows, int D, int d, int dtype,
                 double *Kp);
void orc_score(const double *q_imp, const double *Kp, int Himp, int Hkv, int cap, int d, int n,
               double *s64, float *s32);
int32_t orc_topb64(const double *s, int32_t n, int32_t B, int32_t *T);
int32_t orc_topb(const float *s, int32_t n, int32_t B, int32_t *T);
int32_t orc_expand(const int32_t *T, int32_t nT, int32_t n, int32_t r, int32_t *S);
void orc_mlp(const double *h, const double *W1, const double *W2, int M, int E, int F, int G,
             int Himp, int d, int act, int dtype, double *q_imp);
void orc_buffers(int32_t n, int32_t n_sink, int32_t n_local, int32_t *lo, int32_t *hi);
int32_t orc_select64(const double *s, int32_t n, int32_t B, int32_t r, int32_t n_sink,
                     int32_t n_local, int32_t *T, int32_t *nT, int32_t *S);
int32_t orc_select(const float *s, int32_t n, int32_t B, int32_t r, int32_t n_sink,
                   int32_t n_local, int32_t *T, int32_t *nT, int32_t *S);
void orc_attend(const double *q, const double *K, const double *V, int D, const int32_t *S,
                int32_t nS, double scale, double *out, double *w);
int orc_decode_step(int Hq, int Hkv, int Himp, int D, int d, int cap, int dtype, double *K,
                    double *V, double *Kp, const double *W, const double *k_new,
                    const double *v_new, int n_new, int ctx, const double *q,
                    const double *q_imp, int refresh, int B, int r, int n_sink, int n_local,
                    double scale, int32_t *sel, int32_t *cnt, int32_t *keep_from, int cap_S,
                    double *out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* in [-1, 1), a 64-bit LCG */
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}
static double *rnd(size_t n)
{
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i)
        p[i] = uniform();
    return p;
}

static void decode_run(int Hq, int Hkv, int Himp, int D, int d, int cap, int dtype, int B, int r,
                       int ns, int nl, int ctx0, int steps, int P, int n_new)
{
    const int cap_S = (2 * r + 1) * B + ns + nl < cap ? (2 * r + 1) * B + ns + nl : cap;
    double *K = rnd((size_t)Hkv * cap * D), *V = rnd((size_t)Hkv * cap * D);
    double *W = rnd((size_t)D * d), *Kp = (double *)calloc((size_t)Hkv * cap * d, sizeof(double));
    orc_round(K, K, (int64_t)Hkv * cap * D, dtype);
    orc_round(V, V, (int64_t)Hkv * cap * D, dtype);
    orc_round(W, W, (int64_t)D * d, dtype);
    for (int g = 0; g < Hkv; ++g)
        orc_project(K + (size_t)g * cap * D, W, ctx0, D, d, dtype, Kp + (size_t)g * cap * d);
    int32_t *sel = (int32_t *)calloc((size_t)Himp * cap_S, sizeof(int32_t));
    int32_t cnt[64] = {0}, keep = 0;
    double *out = (double *)malloc((size_t)Hq * D * sizeof(double));
    for (int s = 0; s < steps; ++s) {
        const int ctx = ctx0 + (s + 1) * n_new;
        if (ctx > cap)
            break;
        double *kn = rnd((size_t)Hkv * n_new * D), *vn = rnd((size_t)Hkv * n_new * D);
        double *q = rnd((size_t)Hq * D), *qi = rnd((size_t)Himp * d);
        orc_round(kn, kn, (int64_t)Hkv * n_new * D, dtype);
        orc_round(vn, vn, (int64_t)Hkv * n_new * D, dtype);
        if (orc_decode_step(Hq, Hkv, Himp, D, d, cap, dtype, K, V, Kp, W, kn, vn, n_new, ctx, q,
                            qi, s % P == 0, B, r, ns, nl, 0.125, sel, cnt, &keep, cap_S,
                            out) != 0) {
            fprintf(stderr, "decode step refused a shape\n");
            exit(2);
        }
        free(kn); free(vn); free(q); free(qi);
    }
    free(K); free(V); free(W); free(Kp); free(sel); free(out);
}

int main(void)
{
    /* selection pieces on edge cases: empty rows, B >= n, B = 1, ties, wide radius */
    for (int n = 0; n <= 70; n += 7) {
        double *s = rnd((size_t)n);
        float *sf = (float *)malloc((size_t)(n ? n : 1) * sizeof(float));
        for (int t = 0; t < n; ++t) {
            if (t % 5 == 0)
                s[t] = 0.5; /* ties */
            sf[t] = (float)s[t];
        }
        int32_t *T = (int32_t *)malloc((size_t)(n + 1) * sizeof(int32_t));
        int32_t *S = (int32_t *)malloc((size_t)(n + 1) * sizeof(int32_t));
        for (int B = 1; B <= n + 2; B += 3) {
            int32_t nT = 0, lo, hi;
            orc_topb64(s, n, B, T);
            int32_t k = orc_topb(sf, n, B, T);
            orc_expand(T, k < n ? k : n, n, 3, S);
            orc_buffers(n, 2, 5, &lo, &hi);
            orc_select64(s, n, B, 1, 2, 5, T, &nT, S);
            orc_select(sf, n, B, 40, 0, 0, T, &nT, S);
        }
        free(s); free(sf); free(T); free(S);
    }
    /* scores and attention */
    {
        double *qi = rnd(4 * 16), *Kp = rnd(2 * 100 * 16), *s64 = rnd(4 * 100);
        float s32[4 * 100];
        orc_score(qi, Kp, 4, 2, 100, 16, 100, s64, s32);
        double *q = rnd(64), *K = rnd(50 * 64), *V = rnd(50 * 64), out[64], w[50];
        int32_t S[50];
        for (int k = 0; k < 50; ++k)
            S[k] = k;
        orc_attend(q, K, V, 64, S, 50, 0.125, out, w);
        orc_attend(q, K, V, 64, S, 0, 0.125, out, NULL);
        free(qi); free(Kp); free(s64); free(q); free(K); free(V);
    }
    /* the producer MLP, both activations and dtypes */
    for (int act = 0; act < 2; ++act) {
        double *h = rnd(3 * 32), *W1 = rnd(16 * 32), *W2 = rnd(2 * 4 * 8 * 16);
        double *qo = (double *)malloc(2 * 3 * 4 * 8 * sizeof(double));
        orc_mlp(h, W1, W2, 3, 32, 16, 2, 4, 8, act, act, qo);
        free(h); free(W1); free(W2); free(qo);
    }
    /* fused steps: refresh and reuse, one and several new rows, sink and window */
    decode_run(4, 4, 4, 64, 16, 600, 0, 64, 0, 0, 0, 511, 3, 1, 1);
    decode_run(8, 2, 8, 128, 32, 700, 1, 50, 1, 3, 10, 600, 16, 8, 1);
    decode_run(8, 2, 2, 64, 16, 300, 1, 20, 2, 0, 0, 200, 5, 2, 3);
    decode_run(4, 1, 4, 64, 16, 40, 0, 100, 1, 0, 0, 30, 2, 1, 4); /* B above the context */
    puts("oracle driver done");
    return 0;
}
