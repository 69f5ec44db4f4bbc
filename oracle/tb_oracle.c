/*
 * tb_oracle.c -- plain, single-threaded fp64 reference for the TokenButler
 * sparse-decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no source with the GPU library
 * and must never be used as a fallback for it.
 *
 * Sources (TokenButler: Token Importance is Predictable):
 *   [ABS]  the 2026 abstract on the author page (searcharxiv.com);
 *   [ARCH] the gist.science technical summary, "Methodology > Core Architecture";
 *   [INF]  the gist.science technical summary, "Inference Strategy" and its
 *          "Optimizations" list;
 *   [SIG]  the gist.science technical summary, "Significance".
 *
 * Conventions (readings of the pages; every one is listed in the design notes):
 *   - All inputs arrive as double arrays holding the exact values the GPU
 *     reads (bf16 or fp32 values upcast without rounding).
 *   - One projection matrix W [D][d] per layer, shared by every KV head; no
 *     bias ([ARCH] names a single learned matrix).
 *   - The projected key is the fp64 sum over the head dimension in ascending
 *     order, rounded once (round-to-nearest-even) to the cache dtype.
 *   - The importance score that decides the selection is computed in the
 *     kernel's precision: an fp32 fused multiply-add chain over the d_imp
 *     coordinates in ascending order, starting from +0.  (The pages fix no
 *     precision; a floating-point result that decides an integer -- here the
 *     kept set -- is taken in the same precision on both sides.)  The exact
 *     fp64 dot product is reported beside it, and orc_topb64 / orc_select64
 *     rank those fp64 values: the selection the method defines, which the
 *     tests hold the GPU sets to outside a 1e-6 relative band around the
 *     B-th score (the fp32 chain is the stricter, bit-exact second check).
 *   - Top-B orders tokens by (score descending, index ascending).  -0 and +0
 *     tie.  If B >= n every token is kept.
 *   - Neighbor fetching widens every kept token t to [t-r, t+r] clipped to
 *     [0, n); the union is deduplicated and the budget is not re-applied.
 *   - Sink and local window ([INF], the three buffers): the first n_sink
 *     positions and the last n_local positions of [0, n) are always kept.
 *     The three buffers partition the cache, so the top-B choice is made
 *     among the remaining (middle) positions only; the widened choice is
 *     then united with both ranges.
 *   - Attention is exact softmax attention with logits scaled by the given
 *     softmax scale, computed over the attended set only.
 *   - An empty attended set yields a zero output row.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared tb_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------ */
/* Rounding to the storage dtype                                       */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest bf16 value (ties to even), returned as a
 * double.  bf16 keeps 8 significant bits and fp32's exponent range; below
 * 2^-126 its values are multiples of 2^-133.  Written with frexp/ldexp and
 * nearbyint (which rounds half to even in the default rounding mode). */
static double round_to_bf16(double x)
{
    if (x != x || isinf(x) || x == 0.0)
        return x;
    double ax = fabs(x), r;
    int e;
    double f = frexp(ax, &e); /* ax = f * 2^e, f in [0.5, 1) */
    if (e >= -125) {
        /* normal range: ax >= 2^-126 */
        r = ldexp(nearbyint(ldexp(f, 8)), e - 8);
    } else {
        r = ldexp(nearbyint(ldexp(ax, 133)), -133);
    }
    if (r > 0x1.FEp127)
        r = INFINITY;
    return copysign(r, x);
}

static double round_to_dtype(double x, int dtype)
{
    if (dtype == ORC_BF16)
        return round_to_bf16(x);
    return (double)(float)x; /* C conversion: IEEE round-to-nearest-even */
}

void orc_round(const double *x, double *y, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = round_to_dtype(x[i], dtype);
}

/* ------------------------------------------------------------------ */
/* Key projection ([ARCH] key-cache projection; [INF] batched projection) */
/* ------------------------------------------------------------------ */

/* Kp[r][j] = round( sum_{i=0}^{D-1} K[r][i] * W[i][j] ), r < rows. */
void orc_project(const double *K, const double *W, int64_t rows, int D, int d,
                 int dtype, double *Kp)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i)
                acc += K[r * D + i] * W[(int64_t)i * d + j];
            Kp[r * d + j] = round_to_dtype(acc, dtype);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Importance scores ([ARCH] scoring)                                  */
/* ------------------------------------------------------------------ */

/* KV group scored by importance head i when there are Himp importance heads
 * and Hkv KV heads (Himp is a multiple of Hkv). */
static int imp_group(int i, int Himp, int Hkv) { return (int)((int64_t)i * Hkv / Himp); }

/* For one sequence and t < n (Kp is [Hkv][cap][d]):
 *   s64[i][t] = sum_j q_imp[i][j] * Kp[g(i)][t][j] in fp64, ascending j;
 *   s32[i][t] = the same sum as an fp32 fused multiply-add chain,
 *               acc <- fmaf(q_imp[i][j], Kp[g(i)][t][j], acc), j ascending,
 *               acc starting at +0.  The inputs are fp32/bf16 values, so
 *               converting them to float is exact. */
void orc_score(const double *q_imp, const double *Kp, int Himp, int Hkv, int cap,
               int d, int n, double *s64, float *s32)
{
    for (int i = 0; i < Himp; ++i) {
        int g = imp_group(i, Himp, Hkv);
        for (int t = 0; t < n; ++t) {
            const double *k = Kp + ((int64_t)g * cap + t) * d;
            double acc = 0.0;
            float acc32 = 0.0f;
            for (int j = 0; j < d; ++j) {
                acc += q_imp[(int64_t)i * d + j] * k[j];
                acc32 = fmaf((float)q_imp[(int64_t)i * d + j], (float)k[j], acc32);
            }
            if (s64)
                s64[(int64_t)i * n + t] = acc;
            if (s32)
                s32[(int64_t)i * n + t] = acc32;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Top-B under a fixed budget ([ABS]; [ARCH] scoring)                  */
/* ------------------------------------------------------------------ */

typedef struct {
    double s;
    int32_t t;
} orc_key;

static int orc_key_cmp(const void *a, const void *b)
{
    const orc_key *x = (const orc_key *)a, *y = (const orc_key *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->t > y->t) - (x->t < y->t);
}

/* T = the first min(B, n) tokens in (score desc, index asc) order, written
 * in ascending index order.  Returns |T|.  Scores are compared as doubles:
 * -0 and +0 compare equal, so they tie and the lower index wins. */
int32_t orc_topb64(const double *s, int32_t n, int32_t B, int32_t *T)
{
    if (n <= 0 || B <= 0)
        return 0;
    orc_key *a = (orc_key *)malloc((size_t)n * sizeof(orc_key));
    char *keep = (char *)calloc((size_t)n, 1);
    for (int32_t t = 0; t < n; ++t) {
        a[t].s = s[t];
        a[t].t = t;
    }
    qsort(a, (size_t)n, sizeof(orc_key), orc_key_cmp);
    int32_t m = B < n ? B : n;
    for (int32_t k = 0; k < m; ++k)
        keep[a[k].t] = 1;
    int32_t c = 0;
    for (int32_t t = 0; t < n; ++t)
        if (keep[t])
            T[c++] = t;
    free(keep);
    free(a);
    return c;
}

/* The same ranking of fp32 scores (every float converts to double exactly,
 * so the order is the float order). */
int32_t orc_topb(const float *s, int32_t n, int32_t B, int32_t *T)
{
    if (n <= 0 || B <= 0)
        return 0;
    double *d = (double *)malloc((size_t)n * sizeof(double));
    for (int32_t t = 0; t < n; ++t)
        d[t] = (double)s[t];
    int32_t c = orc_topb64(d, n, B, T);
    free(d);
    return c;
}

/* ------------------------------------------------------------------ */
/* Neighbor fetching ([INF] "Prediction Interval & Neighbor Fetching") */
/* ------------------------------------------------------------------ */

/* S = sorted union over t in T of [max(0, t-r), min(n-1, t+r)].  Returns |S|. */
int32_t orc_expand(const int32_t *T, int32_t nT, int32_t n, int32_t r, int32_t *S)
{
    if (n <= 0)
        return 0;
    char *in = (char *)calloc((size_t)n, 1);
    for (int32_t k = 0; k < nT; ++k) {
        int32_t lo = T[k] - r < 0 ? 0 : T[k] - r;
        int32_t hi = T[k] + r > n - 1 ? n - 1 : T[k] + r;
        for (int32_t t = lo; t <= hi; ++t)
            in[t] = 1;
    }
    int32_t c = 0;
    for (int32_t t = 0; t < n; ++t)
        if (in[t])
            S[c++] = t;
    free(in);
    return c;
}

/* ------------------------------------------------------------------ */
/* Importance-query producer ([ARCH] Query Prediction)                 */
/* ------------------------------------------------------------------ */

#define ORC_ACT_RELU 0
#define ORC_ACT_SILU 1

static double orc_act(double x, int act)
{
    if (act == ORC_ACT_SILU)
        return x / (1.0 + exp(-x));
    return x > 0.0 ? x : 0.0;
}

/*
 * The lightweight MLP on the producer layer's hidden states:
 *   u[m][f] = round_dtype( act( sum_e h[m][e] * W1[f][e] ) )      (fp64 sum)
 *   y[m][n] = round_dtype( sum_f u[m][f] * W2[n][f] )             (fp64 sum)
 * with n = (g * Himp + i) * d + j, written slot-major:
 *   q_imp[g][m][i][j] = y[m][n],  G = N / (Himp * d) slots.
 * Weights are stored output-major ([F][E] and [N][F]).  No biases.
 */
void orc_mlp(const double *h, const double *W1, const double *W2, int M, int E, int F, int G,
             int Himp, int d, int act, int dtype, double *q_imp)
{
    const int N = G * Himp * d;
    double *u = (double *)malloc((size_t)M * F * sizeof(double));
    for (int m = 0; m < M; ++m)
        for (int f = 0; f < F; ++f) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e)
                acc += h[(int64_t)m * E + e] * W1[(int64_t)f * E + e];
            u[(int64_t)m * F + f] = round_to_dtype(orc_act(acc, act), dtype);
        }
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int f = 0; f < F; ++f)
                acc += u[(int64_t)m * F + f] * W2[(int64_t)n * F + f];
            const int g = n / (Himp * d), r = n % (Himp * d);
            q_imp[((int64_t)g * M + m) * Himp * d + r] = round_to_dtype(acc, dtype);
        }
    free(u);
}

/* ------------------------------------------------------------------ */
/* The three buffers ([INF]: sink, local window, important)            */
/* ------------------------------------------------------------------ */

/* Bounds of the middle region [*lo, *hi) of a context of n tokens: the sink
 * is [0, *lo), the local window [*hi, n). */
void orc_buffers(int32_t n, int32_t n_sink, int32_t n_local, int32_t *lo, int32_t *hi)
{
    int32_t a = n_sink < n ? n_sink : n;
    int32_t b = n - n_local;
    if (b < a)
        b = a;
    *lo = a;
    *hi = b;
}

/* One head's kept set S over a context of n tokens (fp64 scores s): the
 * important buffer is the top-B tokens of the middle region (T, written to
 * T when not NULL), widened by r; S is its union with the sink and the local
 * window, in ascending order.  Returns |S|; *nT receives |T|. */
int32_t orc_select64(const double *s, int32_t n, int32_t B, int32_t r, int32_t n_sink,
                     int32_t n_local, int32_t *T, int32_t *nT, int32_t *S)
{
    if (n <= 0) {
        *nT = 0;
        return 0;
    }
    int32_t lo, hi;
    orc_buffers(n, n_sink, n_local, &lo, &hi);
    int32_t *Tm = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    int32_t *E = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    /* 1. important buffer: top-B of the middle region, back in context positions */
    int32_t m = orc_topb64(s + lo, hi - lo, B, Tm);
    for (int32_t k = 0; k < m; ++k)
        Tm[k] += lo;
    /* 2. neighbor fetching */
    int32_t ne = orc_expand(Tm, m, n, r, E);
    /* 3. union with the sink [0, lo) and the local window [hi, n) */
    char *in = (char *)calloc((size_t)n, 1);
    for (int32_t k = 0; k < ne; ++k)
        in[E[k]] = 1;
    for (int32_t t = 0; t < lo; ++t)
        in[t] = 1;
    for (int32_t t = hi; t < n; ++t)
        in[t] = 1;
    int32_t c = 0;
    for (int32_t t = 0; t < n; ++t)
        if (in[t])
            S[c++] = t;
    if (T)
        memcpy(T, Tm, (size_t)m * sizeof(int32_t));
    *nT = m;
    free(in);
    free(E);
    free(Tm);
    return c;
}

/* orc_select on fp32 scores (ranked as their exact double values). */
int32_t orc_select(const float *s, int32_t n, int32_t B, int32_t r, int32_t n_sink,
                   int32_t n_local, int32_t *T, int32_t *nT, int32_t *S)
{
    double *d = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int32_t t = 0; t < n; ++t)
        d[t] = (double)s[t];
    int32_t c = orc_select64(d, n, B, r, n_sink, n_local, T, nT, S);
    free(d);
    return c;
}

/* ------------------------------------------------------------------ */
/* Attention over the selected rows only ([ABS]; [SIG])                */
/* ------------------------------------------------------------------ */

/* out[i] = sum_k w_k V[S[k]][i],  w = softmax_k( scale * q . K[S[k]] ).
 * K and V are one KV head's rows [*][D].  Two passes (max, then exp/sum),
 * ascending k.  w (nullable) receives the weights.  nS == 0 gives out = 0. */
void orc_attend(const double *q, const double *K, const double *V, int D,
                const int32_t *S, int32_t nS, double scale, double *out, double *w)
{
    for (int i = 0; i < D; ++i)
        out[i] = 0.0;
    if (nS <= 0)
        return;
    double *z = (double *)malloc((size_t)nS * sizeof(double));
    double zmax = -INFINITY;
    for (int32_t k = 0; k < nS; ++k) {
        const double *kr = K + (int64_t)S[k] * D;
        double dot = 0.0;
        for (int i = 0; i < D; ++i)
            dot += q[i] * kr[i];
        z[k] = scale * dot;
        if (z[k] > zmax)
            zmax = z[k];
    }
    double denom = 0.0;
    for (int32_t k = 0; k < nS; ++k) {
        z[k] = exp(z[k] - zmax);
        denom += z[k];
    }
    for (int32_t k = 0; k < nS; ++k) {
        double wk = z[k] / denom;
        if (w)
            w[k] = wk;
        const double *vr = V + (int64_t)S[k] * D;
        for (int i = 0; i < D; ++i)
            out[i] += wk * vr[i];
    }
    free(z);
}

/* ------------------------------------------------------------------ */
/* One decode step of one sequence ([INF]: projection batching,        */
/* prediction interval, neighbor fetching; [ABS]: selection + attention) */
/* ------------------------------------------------------------------ */

/*
 * Layouts (one sequence):
 *   K, V   [Hkv][cap][D]    updated in place with the appended rows
 *   Kp     [Hkv][cap][d]    updated in place with their projections
 *   W      [D][d]
 *   k_new, v_new [Hkv][n_new][D] (may be NULL when n_new == 0)
 *   q      [Hq][D]
 *   q_imp  [Himp][d]        read only when refresh != 0
 *   sel    [Himp][cap_S], cnt [Himp], keep_from [1]: the selection state
 *   out    [Hq][D]
 *
 * ctx is the context length after the append; the new rows occupy
 * [ctx - n_new, ctx).  On a refresh step every importance head is scored over
 * [0, ctx), its kept set is taken (orc_select: top-B of the middle region
 * widened by radius r, plus the sink and the local window), the result is
 * stored in sel/cnt and keep_from is set to ctx - n_new.  Every step then
 * attends, for query head h, over sel[imp(h)] united with [keep_from, ctx).
 * Returns 0, or -1 when a stored set would overflow cap_S.
 */
int orc_decode_step(int Hq, int Hkv, int Himp, int D, int d, int cap, int dtype,
                    double *K, double *V, double *Kp, const double *W,
                    const double *k_new, const double *v_new, int n_new, int ctx,
                    const double *q, const double *q_imp, int refresh, int B, int r,
                    int n_sink, int n_local, double scale, int32_t *sel, int32_t *cnt,
                    int32_t *keep_from, int cap_S, double *out)
{
    /* 1. append the new rows and project their keys */
    for (int j = 0; j < n_new; ++j) {
        int pos = ctx - n_new + j;
        for (int g = 0; g < Hkv; ++g) {
            double *kr = K + ((int64_t)g * cap + pos) * D;
            double *vr = V + ((int64_t)g * cap + pos) * D;
            memcpy(kr, k_new + ((int64_t)g * n_new + j) * D, (size_t)D * sizeof(double));
            memcpy(vr, v_new + ((int64_t)g * n_new + j) * D, (size_t)D * sizeof(double));
            orc_project(kr, W, 1, D, d, dtype, Kp + ((int64_t)g * cap + pos) * d);
        }
    }
    /* 2. on a refresh step: score, keep top-B, widen, store */
    if (refresh) {
        float *s = (float *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(float));
        int32_t *T = (int32_t *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(int32_t));
        int32_t *S = (int32_t *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(int32_t));
        for (int i = 0; i < Himp; ++i) {
            /* score head i alone: pass its query row and view it as 1 head */
            int g = imp_group(i, Himp, Hkv);
            orc_score(q_imp + (int64_t)i * d, Kp + (int64_t)g * cap * d, 1, 1, cap, d, ctx,
                      NULL, s);
            int32_t nT = 0;
            int32_t nS = orc_select(s, ctx, B, r, n_sink, n_local, T, &nT, S);
            if (nS > cap_S) {
                free(s);
                free(T);
                free(S);
                return -1;
            }
            memcpy(sel + (int64_t)i * cap_S, S, (size_t)nS * sizeof(int32_t));
            cnt[i] = nS;
        }
        keep_from[0] = ctx - n_new;
        free(s);
        free(T);
        free(S);
    }
    /* 3. attend over the stored set plus the rows appended since the refresh */
    char *in = (char *)malloc((size_t)(ctx > 0 ? ctx : 1));
    int32_t *A = (int32_t *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(int32_t));
    for (int h = 0; h < Hq; ++h) {
        int g = (int)((int64_t)h * Hkv / Hq);
        int i = (int)((int64_t)h * Himp / Hq);
        memset(in, 0, (size_t)(ctx > 0 ? ctx : 1));
        for (int32_t k = 0; k < cnt[i]; ++k)
            if (sel[(int64_t)i * cap_S + k] < ctx)
                in[sel[(int64_t)i * cap_S + k]] = 1;
        for (int t = keep_from[0] < 0 ? 0 : keep_from[0]; t < ctx; ++t)
            in[t] = 1;
        int32_t nA = 0;
        for (int t = 0; t < ctx; ++t)
            if (in[t])
                A[nA++] = t;
        orc_attend(q + (int64_t)h * D, K + (int64_t)g * cap * D, V + (int64_t)g * cap * D, D,
                   A, nA, scale, out + (int64_t)h * D, NULL);
    }
    free(in);
    free(A);
    return 0;
}
