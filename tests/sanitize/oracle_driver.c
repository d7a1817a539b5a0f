/*
 * Driver for a sanitizer build of the fp64 oracle (oracle/oracle.c, built
 * without OpenMP with the address and undefined-behaviour sanitizers).  It
 * calls every exported function on small seeded inputs -- truncated lists,
 * fp32 and bf16 weights, dense and thresholded attention rows, invalid
 * arguments -- and checks the invariants any correct result has (ascending
 * lists, positive soft-threshold values, counts within range, finite
 * outputs), so that the sanitizers see every loop and buffer of the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_norm_quantile(double p);
double oracle_gelu_tanh(double v);
double oracle_softplus(double v);
double oracle_threshold_z(int64_t k, int64_t d);
int oracle_stat_topk(const float *x, int64_t rows, int64_t d, int64_t ldx, int64_t k, int64_t cap, double *vals,
                     int32_t *idx, int32_t *counts, double *theta, double *mean, double *sd);
int oracle_spark_ffn(int64_t d_model, int64_t d_ff, int64_t r, int64_t k, int wdtype, const void *k1t,
                     const void *k2t, const void *v, int qdtype, const void *q, int64_t T, double *y,
                     int32_t *counts, double *h, int32_t *idx, double *m, int64_t cap, double *theta, double *mean,
                     double *sd);
int oracle_decode_stack(int64_t d_model, int64_t d_ff, int64_t r, int64_t k, int wdtype, int n_layers,
                        const void *const *k1t, const void *const *k2t, const void *const *v, const float *q0,
                        int64_t T, double eps, double *y, int32_t *counts, double *q_trace);
int oracle_spark_attn_decode(int dtype, const void *q, const void *k1, const void *k2, const void *v, int64_t Hq,
                             int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double *out,
                             int32_t *counts, double *theta, double *scores);
double oracle_huber_relu(double u, double delta);
double oracle_huber_relu_grad(double u, double delta);
int oracle_stat_topk_huber_forward(const float *x, int64_t rows, int64_t d, int64_t k, double delta, double *y,
                                   double *theta);
int oracle_stat_topk_huber_backward(const float *x, const float *dy, int64_t rows, int64_t d, int64_t k,
                                    double delta, double *dx);
int oracle_spark_attn_prefill(int dtype, const void *q, const void *k1, const void *k2, const void *v, int64_t T,
                              int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, double *out,
                              int32_t *counts, double *theta);

static int failures = 0;
#define EXPECT(c)                                                                 \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);      \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static uint64_t state = 88172645463325252ull;
static double uniform(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return ((double)(state >> 11) + 0.5) / 9007199254740992.0;
}
static double normal(void) { return sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform()); }

static float *f32s(int64_t n, double scale)
{
    float *a = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) a[i] = (float)(scale * normal());
    return a;
}
static uint16_t *bf16s(int64_t n, double scale)
{
    uint16_t *a = malloc(sizeof(uint16_t) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)(scale * normal());
        uint32_t u;
        memcpy(&u, &f, 4);
        a[i] = (uint16_t)(u >> 16); /* truncation is enough for test inputs */
    }
    return a;
}

static void check_list(const int32_t *idx, const double *vals, int64_t n, int64_t d)
{
    for (int64_t e = 0; e < n; ++e) {
        EXPECT(idx[e] >= 0 && idx[e] < d);
        if (e) EXPECT(idx[e] > idx[e - 1]);
        if (vals) EXPECT(vals[e] > 0.0);
    }
}

int main(void)
{
    /* scalars */
    for (int i = 1; i < 1000; ++i) EXPECT(isfinite(oracle_norm_quantile(i / 1000.0)));
    EXPECT(isnan(oracle_norm_quantile(0.0)) || isinf(oracle_norm_quantile(0.0)) || oracle_norm_quantile(0.0) < -30);
    EXPECT(oracle_gelu_tanh(0.0) == 0.0 && isfinite(oracle_softplus(-800.0)) && isfinite(oracle_softplus(800.0)));

    /* statistical top-k, list capacity below the counts */
    {
        const int64_t rows = 9, d = 1000, k = 80, cap = 50;
        float *x = f32s(rows * d, 1.0);
        double *vals = malloc(sizeof(double) * rows * cap), th[9], mu[9], sd[9];
        int32_t *idx = malloc(sizeof(int32_t) * rows * cap), counts[9];
        EXPECT(oracle_stat_topk(x, rows, d, d, k, cap, vals, idx, counts, th, mu, sd) == 0);
        for (int64_t r = 0; r < rows; ++r) {
            EXPECT(counts[r] > 0 && counts[r] < d);
            check_list(idx + r * cap, vals + r * cap, counts[r] < cap ? counts[r] : cap, d);
        }
        EXPECT(oracle_stat_topk(x, rows, d, d - 1, k, cap, vals, idx, counts, th, mu, sd) == -1);
        EXPECT(oracle_stat_topk(x, rows, d, d, d, cap, vals, idx, counts, th, mu, sd) == -1);
        free(x), free(vals), free(idx);
    }

    /* one FFN layer, fp32 and bf16 weights */
    for (int wd = 0; wd < 2; ++wd) {
        const int64_t dm = 64, dff = 256, r = 32, k = 20, T = 3, cap = 10;
        void *k1 = wd ? (void *)bf16s(dff * r, 0.18) : (void *)f32s(dff * r, 0.18);
        void *k2 = wd ? (void *)bf16s(dff * (dm - r), 0.18) : (void *)f32s(dff * (dm - r), 0.18);
        void *v = wd ? (void *)bf16s(dff * dm, 0.06) : (void *)f32s(dff * dm, 0.06);
        float *q = f32s(T * dm, 1.0);
        double *y = malloc(sizeof(double) * T * dm), *h = malloc(sizeof(double) * T * dff),
               *m = malloc(sizeof(double) * T * cap), th[3], mu[3], sd[3];
        int32_t counts[3], *idx = malloc(sizeof(int32_t) * T * cap);
        EXPECT(oracle_spark_ffn(dm, dff, r, k, wd, k1, k2, v, 0, q, T, y, counts, h, idx, m, cap, th, mu, sd) == 0);
        for (int64_t t = 0; t < T; ++t) {
            check_list(idx + t * cap, m + t * cap, counts[t] < cap ? counts[t] : cap, dff);
            for (int64_t c = 0; c < dm; ++c) EXPECT(isfinite(y[t * dm + c]));
        }
        EXPECT(oracle_spark_ffn(dm, dff, dm, k, wd, k1, k2, v, 0, q, T, y, counts, h, idx, m, cap, th, mu, sd) == -1);
        /* the stack: three layers of the same weights */
        const void *K1[3] = {k1, k1, k1}, *K2[3] = {k2, k2, k2}, *V[3] = {v, v, v};
        double *qt = malloc(sizeof(double) * T * 3 * dm);
        int32_t sc[9];
        EXPECT(oracle_decode_stack(dm, dff, r, k, wd, 3, K1, K2, V, q, T, 1e-6, y, sc, qt) == 0);
        for (int i = 0; i < 9; ++i) EXPECT(sc[i] >= 0 && sc[i] <= dff);
        free(k1), free(k2), free(v), free(q), free(y), free(h), free(m), free(idx), free(qt);
    }

    /* attention decode (dense and thresholded) and causal prefill */
    {
        const int64_t Hq = 4, Hkv = 2, hd = 32, r = 16, n = 100;
        uint16_t *q = bf16s(Hq * hd, 0.18), *k1 = bf16s(Hkv * n * r, 0.18), *k2 = bf16s(Hkv * n * (hd - r), 0.18),
                 *v = bf16s(Hkv * n * hd, 0.18);
        double *out = malloc(sizeof(double) * Hq * hd), th[4], *sc = malloc(sizeof(double) * Hq * n);
        int32_t cnt[4];
        EXPECT(oracle_spark_attn_decode(1, q, k1, k2, v, Hq, Hkv, n, hd, r, 20, out, cnt, th, sc) == 0);
        for (int h = 0; h < Hq; ++h) EXPECT(cnt[h] > 0 && cnt[h] <= n && !isnan(th[h]));
        EXPECT(oracle_spark_attn_decode(1, q, k1, k2, v, Hq, Hkv, n, hd, r, 200, out, cnt, th, sc) == 0);
        for (int h = 0; h < Hq; ++h) EXPECT(cnt[h] == n && isnan(th[h]));
        EXPECT(oracle_spark_attn_decode(1, q, k1, k2, v, Hq, 3, n, hd, r, 20, out, cnt, th, sc) == -1);
        const int64_t T = 40;
        uint16_t *qp = bf16s(T * Hq * hd, 0.18);
        double *op = malloc(sizeof(double) * T * Hq * hd), *tp = malloc(sizeof(double) * T * Hq);
        int32_t *cp = malloc(sizeof(int32_t) * T * Hq);
        EXPECT(oracle_spark_attn_prefill(1, qp, k1, k2, v, T, Hq, Hkv, hd, r, 8, op, cp, tp) == 0);
        for (int64_t i = 0; i < T * Hq; ++i) EXPECT(cp[i] > 0 && cp[i] <= i / Hq + 1 && isfinite(op[i * hd]));
        free(q), free(k1), free(k2), free(v), free(out), free(sc), free(qp), free(op), free(tp), free(cp);
    }
    /* training side: Huber-smoothed statistical top-k, forward and gradient */
    {
        const int64_t rows = 5, d = 300, k = 25;
        float *x = f32s(rows * d, 1.0), *dy = f32s(rows * d, 1.0);
        double *y = malloc(sizeof(double) * rows * d), *dx = malloc(sizeof(double) * rows * d), th[5];
        EXPECT(oracle_stat_topk_huber_forward(x, rows, d, k, 0.1, y, th) == 0);
        EXPECT(oracle_stat_topk_huber_backward(x, dy, rows, d, k, 0.1, dx) == 0);
        for (int64_t r = 0; r < rows; ++r) {
            double s = 0.0, m = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                EXPECT(y[r * d + i] >= 0.0 && isfinite(dx[r * d + i]));
                s += dx[r * d + i];
                m = fmax(m, fabs(dx[r * d + i]));
            }
            EXPECT(fabs(s) <= 1e-9 * (1.0 + m * d));
        }
        EXPECT(oracle_stat_topk_huber_forward(x, rows, d, k, 0.0, y, th) == -1);
        EXPECT(oracle_stat_topk_huber_backward(x, dy, rows, d, d, 0.1, dx) == -1);
        EXPECT(oracle_huber_relu(-1.0, 0.5) == 0.0 && oracle_huber_relu_grad(2.0, 0.5) == 1.0);
        free(x), free(dy), free(y), free(dx);
    }
    printf("oracle driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
