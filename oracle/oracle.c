/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the Spark FFN layer, the
 * statistical top-k operator and Spark attention (decode and causal prefill).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline use it.  It shares no code, header, table or constant with the
 * HIP library under attention_spark_ffn_amd/csrc.
 *
 * Sources (the pages are the Spark Transformer reading notes, "Spark
 * Transformer: Reactivating Sparsity in FFN and Attention", section
 * "方法详解 / 关键设计", and the arXiv abstract of the same paper):
 *   - Spark FFN formula: Spark-FFN(q) = V (sigma(Top_k(K1^T q[:r])) (.) (K2^T q[r:]))
 *     with q split at r, only the selected K2 columns and V rows used
 *     (notes, "Spark FFN" item of the key-design section).
 *   - Statistical top-k: theta(x,k) = mean(x) + std(x) Q(1-k/d), Q the
 *     standard-normal quantile, followed by the soft-threshold
 *     max{x - theta, 0} (notes, "Statistical Top-k" item).
 *   - Spark attention: same form as the FFN, key dims split into a
 *     predictor part K1 and a compute part K2, sigma1 = softmax,
 *     sigma2 = softplus, about k_attn = 256 attended tokens
 *     (notes, "Spark Attention" item; abstract).
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes of the repository):
 *   std is the population std (1/d), as in LayerNorm, which the notes
 *   compare the operator to; selection is strict (x > theta); the compacted
 *   index list is ascending; the value kept for a selected entry is the
 *   soft-threshold output x - theta; sigma of the FFN is the tanh form of
 *   GELU; V is stored [d_ff][d_model] and its rows are neurons; attention
 *   uses no 1/sqrt(hd) factor, softmax runs over the selected set only,
 *   query head h reads KV head h / (Hq/Hkv), and when n_ctx <= k_attn all
 *   tokens are attended; in a causal prefill the query of position t
 *   attends over positions 0..t with its own threshold.  An empty selected set gives a zero output.
 *
 * Arithmetic: every stored input (fp32, or bf16 widened exactly) is read as
 * is and all arithmetic is IEEE fp64 in plain loops, summing in ascending
 * index order.  OpenMP only splits independent rows/neurons/columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };

/* Exact widening of one stored element to fp64. */
static double ld(const void *base, int dtype, int64_t i)
{
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Standard-normal quantile Q(p), the function the threshold formula of the
 * statistical top-k uses.  Written from Wichura's algorithm AS 241
 * (PPND16, Applied Statistics 37 (1988) 477-484): a rational function of
 * (p-1/2) in the centre, and of sqrt(-log(min(p,1-p))) in the two tail
 * ranges, with the published coefficients.
 */
double oracle_norm_quantile(double p)
{
    if (!(p > 0.0 && p < 1.0))
        return p == 0.0 ? -INFINITY : (p == 1.0 ? INFINITY : NAN);
    double q = p - 0.5;
    if (fabs(q) <= 0.425) {
        double t = 0.180625 - q * q;
        double num = ((((((2.5090809287301226727e3 * t + 3.3430575583588128105e4) * t +
                          6.7265770927008700853e4) * t + 4.5921953931549871457e4) * t +
                        1.3731693765509461125e4) * t + 1.9715909503065514427e3) * t +
                      1.3314166789178437745e2) * t + 3.3871328727963666080e0;
        double den = ((((((5.2264952788528545610e3 * t + 2.8729085735721942674e4) * t +
                          3.9307895800092710610e4) * t + 2.1213794301586595867e4) * t +
                        5.3941960214247511077e3) * t + 6.8718700749205790830e2) * t +
                      4.2313330701600911252e1) * t + 1.0;
        return q * num / den;
    }
    double t = q < 0.0 ? p : 1.0 - p;
    t = sqrt(-log(t));
    double v;
    if (t <= 5.0) {
        t -= 1.6;
        double num = ((((((7.74545014278341407640e-4 * t + 2.27238449892691845833e-2) * t +
                          2.41780725177450611770e-1) * t + 1.27045825245236838258e0) * t +
                        3.64784832476320460504e0) * t + 5.76949722146069140550e0) * t +
                      4.63033784615654529590e0) * t + 1.42343711074968357734e0;
        double den = ((((((1.05075007164441684324e-9 * t + 5.47593808499534494600e-4) * t +
                          1.51986665636164571966e-2) * t + 1.48103976427480074590e-1) * t +
                        6.89767334985100004550e-1) * t + 1.67638483018380384940e0) * t +
                      2.05319162663775882187e0) * t + 1.0;
        v = num / den;
    } else {
        t -= 5.0;
        double num = ((((((2.01033439929228813265e-7 * t + 2.71155556874348757815e-5) * t +
                          1.24266094738807843860e-3) * t + 2.65321895265761230930e-2) * t +
                        2.96560571828504891230e-1) * t + 1.78482653991729133580e0) * t +
                      5.46378491116411436990e0) * t + 6.65790464350110377720e0;
        double den = ((((((2.04426310338993978564e-15 * t + 1.42151175831644588870e-7) * t +
                          1.84631831751005468180e-5) * t + 7.86869131145613259100e-4) * t +
                        1.48753612908506148525e-2) * t + 1.36929880922735805310e-1) * t +
                      5.99832206555887937690e-1) * t + 1.0;
        v = num / den;
    }
    return q < 0.0 ? -v : v;
}

/* sigma of the Spark FFN: the tanh form of GELU,
 * 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))). */
double oracle_gelu_tanh(double v)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

/* sigma2 of Spark attention: softplus log(1 + e^v), written in the
 * overflow-free form max(v,0) + log1p(e^-|v|). */
double oracle_softplus(double v)
{
    return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

/*
 * Statistical top-k of one fp64 row (threshold formula and soft-threshold of
 * the "Statistical Top-k" item).  Writes mean, std, theta; stores the
 * ascending list of i with x_i > theta and m_i = x_i - theta, keeping the
 * first `cap` of them; returns the true count.
 */
static int64_t stat_topk_row(const double *x, int64_t d, double z, double *mean_out, double *std_out,
                             double *theta_out, int32_t *idx, double *m, int64_t cap)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i)
        s += x[i];
    double mean = s / (double)d;
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i)
        ss += (x[i] - mean) * (x[i] - mean);
    double sd = sqrt(ss / (double)d);
    double theta = mean + sd * z;
    int64_t count = 0;
    for (int64_t i = 0; i < d; ++i) {
        if (x[i] > theta) {
            if (count < cap) {
                if (idx) idx[count] = (int32_t)i;
                if (m) m[count] = x[i] - theta;
            }
            ++count;
        }
    }
    if (mean_out) *mean_out = mean;
    if (std_out) *std_out = sd;
    if (theta_out) *theta_out = theta;
    return count;
}

/* z = Q(1 - k/d) as the threshold formula states it. */
double oracle_threshold_z(int64_t k, int64_t d)
{
    return oracle_norm_quantile(1.0 - (double)k / (double)d);
}

/*
 * Standalone statistical top-k over `rows` fp32 rows of length d (row stride
 * ldx).  vals/idx are [rows][cap]; counts, theta, mean, std are [rows].
 * Any of vals, idx, theta, mean, std may be NULL.  Returns 0, or -1 on bad
 * arguments.
 */
int oracle_stat_topk(const float *x, int64_t rows, int64_t d, int64_t ldx, int64_t k, int64_t cap,
                     double *vals, int32_t *idx, int32_t *counts, double *theta, double *mean, double *sd)
{
    if (!x || !counts || rows < 0 || d <= 0 || ldx < d || k <= 0 || k >= d || cap < 0)
        return -1;
    const double z = oracle_threshold_z(k, d);
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t i = 0; i < d; ++i)
                row[i] = (double)x[r * ldx + i];
            double mu, s, th;
            int64_t c = stat_topk_row(row, d, z, &mu, &s, &th, idx ? idx + r * cap : NULL,
                                      vals ? vals + r * cap : NULL, cap);
            counts[r] = (int32_t)c;
            if (theta) theta[r] = th;
            if (mean) mean[r] = mu;
            if (sd) sd[r] = s;
        }
        free(row);
    }
    return 0;
}

/*
 * Training side of the statistical top-k (notes, "Statistical Top-k" item,
 * differentiability bullet: with Huber smoothing the operator becomes
 * continuously differentiable).  The pages name the smoothing but do not
 * print it; the reading taken here replaces the soft-threshold max{u, 0},
 * u = x - theta, by its Huber smoothing of width delta > 0,
 *     h(u) = 0 (u <= 0),  u^2 / (2 delta) (0 < u < delta),  u - delta / 2 (u >= delta),
 * the integral from 0 to u of min(max(t / delta, 0), 1): a quadratic joint in
 * place of the kink, continuously differentiable, within delta / 2 of
 * max{u, 0} and equal to it as delta -> 0.  theta is the same
 * mean + std * Q(1 - k/d) as in the forward operator, and its dependence on
 * every x_j is part of the gradient.
 */
double oracle_huber_relu(double u, double delta)
{
    if (u <= 0.0) return 0.0;
    if (u < delta) return u * u / (2.0 * delta);
    return u - 0.5 * delta;
}

/* h'(u) = min(max(u / delta, 0), 1). */
double oracle_huber_relu_grad(double u, double delta)
{
    if (u <= 0.0) return 0.0;
    if (u < delta) return u / delta;
    return 1.0;
}

/* Mean and population std of one fp32 row, two passes in ascending order. */
static void row_moments(const float *x, int64_t d, double *mean, double *sd)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i)
        s += (double)x[i];
    const double mu = s / (double)d;
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i)
        ss += ((double)x[i] - mu) * ((double)x[i] - mu);
    *mean = mu;
    *sd = sqrt(ss / (double)d);
}

/*
 * Forward: y[r][i] = h(x[r][i] - theta_r) for every entry (a dense [rows][d]
 * result, zero below the threshold).  theta [rows] may be NULL.  Returns 0,
 * or -1 on bad arguments.
 */
int oracle_stat_topk_huber_forward(const float *x, int64_t rows, int64_t d, int64_t k, double delta, double *y,
                                   double *theta)
{
    if (!x || !y || rows < 0 || d <= 0 || k <= 0 || k >= d || !(delta > 0.0))
        return -1;
    const double z = oracle_threshold_z(k, d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double mu, sd;
        row_moments(x + r * d, d, &mu, &sd);
        const double th = mu + sd * z;
        for (int64_t i = 0; i < d; ++i)
            y[r * d + i] = oracle_huber_relu((double)x[r * d + i] - th, delta);
        if (theta) theta[r] = th;
    }
    return 0;
}

/*
 * Backward: given dy = dL/dy, dx = dL/dx by the chain rule through
 * y_i = h(x_i - theta(x)):
 *     a_i = dy_i h'(x_i - theta),   A = sum_i a_i,
 *     d theta / d x_j = 1/d + z (x_j - mean) / (d std)   (d mean/dx_j = 1/d,
 *                                   d std/dx_j = (x_j - mean) / (d std)),
 *     dx_j = a_j - A d theta / d x_j.
 * A row with zero spread has x_i - theta = 0 everywhere, so a = 0, A = 0 and
 * dx = 0 (its std term, 0/0, is never formed).  Returns 0, or -1 on bad
 * arguments.
 */
int oracle_stat_topk_huber_backward(const float *x, const float *dy, int64_t rows, int64_t d, int64_t k,
                                    double delta, double *dx)
{
    if (!x || !dy || !dx || rows < 0 || d <= 0 || k <= 0 || k >= d || !(delta > 0.0))
        return -1;
    const double z = oracle_threshold_z(k, d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double mu, sd;
        row_moments(x + r * d, d, &mu, &sd);
        const double th = mu + sd * z;
        double A = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            const double a = (double)dy[r * d + i] * oracle_huber_relu_grad((double)x[r * d + i] - th, delta);
            dx[r * d + i] = a;
            A += a;
        }
        for (int64_t j = 0; j < d; ++j) {
            double dth = 1.0 / (double)d;
            if (sd > 0.0) dth += z * ((double)x[r * d + j] - mu) / ((double)d * sd);
            dx[r * d + j] -= A * dth;
        }
    }
    return 0;
}

/*
 * One Spark FFN evaluation for one token, q given in fp64 (length d_model).
 * Weights in the stored layouts: k1t [d_ff][r] (K1 transposed: row i is the
 * predictor key of neuron i), k2t [d_ff][d_model-r] (K2 transposed), v
 * [d_ff][d_model]; dtype OR_F32 or OR_BF16.  Writes y [d_model]; optional
 * outputs: h [d_ff] (predictor scores), idx/m [cap] (selected neurons and
 * soft-threshold values), theta/mean/std.  Returns the selected count.
 * Threads split the neuron loop of the predictor and the column loop of the
 * V accumulation; every sum runs in ascending index order.
 */
static int64_t ffn_token(int64_t d_model, int64_t d_ff, int64_t r, double z, int wdtype, const void *k1t,
                         const void *k2t, const void *v, const double *q, double *y, double *h_out,
                         int32_t *idx_out, double *m_out, int64_t cap, double *theta_out, double *mean_out,
                         double *std_out)
{
    const int64_t rc = d_model - r;
    double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
    int32_t *S = (int32_t *)malloc(sizeof(int32_t) * (size_t)d_ff);
    double *m = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *c = (double *)malloc(sizeof(double) * (size_t)d_ff);

    /* predictor: h_i = sum_{j<r} K1[j][i] q[j] */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_ff; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < r; ++j)
            s += ld(k1t, wdtype, i * r + j) * q[j];
        h[i] = s;
    }
    double th, mu, sd;
    int64_t n = stat_topk_row(h, d_ff, z, &mu, &sd, &th, S, m, d_ff);

    /* gated value of each selected neuron: c_i = GELU(m_i) * (K2[:,i] . q[r:]) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = S[t];
        double g = 0.0;
        for (int64_t j = 0; j < rc; ++j)
            g += ld(k2t, wdtype, i * rc + j) * q[r + j];
        c[t] = oracle_gelu_tanh(m[t]) * g;
    }
    /* y = sum over selected neurons (ascending) of c_i V[i][:] */
#pragma omp parallel for schedule(static)
    for (int64_t col = 0; col < d_model; ++col) {
        double s = 0.0;
        for (int64_t t = 0; t < n; ++t)
            s += c[t] * ld(v, wdtype, (int64_t)S[t] * d_model + col);
        y[col] = s;
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)d_ff);
    for (int64_t t = 0; t < n && t < cap; ++t) {
        if (idx_out) idx_out[t] = S[t];
        if (m_out) m_out[t] = m[t];
    }
    if (theta_out) *theta_out = th;
    if (mean_out) *mean_out = mu;
    if (std_out) *std_out = sd;
    free(h);
    free(S);
    free(m);
    free(c);
    return n;
}

/*
 * Spark FFN over T independent tokens of one layer.  q is [T][d_model] of
 * dtype qdtype (OR_F32 or OR_BF16); y [T][d_model].  Optional: counts [T],
 * h [T][d_ff], idx/m [T][cap], theta/mean/std [T].
 */
int oracle_spark_ffn(int64_t d_model, int64_t d_ff, int64_t r, int64_t k, int wdtype, const void *k1t,
                     const void *k2t, const void *v, int qdtype, const void *q, int64_t T, double *y,
                     int32_t *counts, double *h, int32_t *idx, double *m, int64_t cap, double *theta,
                     double *mean, double *sd)
{
    if (!k1t || !k2t || !v || !q || !y || T < 0 || r <= 0 || r >= d_model || k <= 0 || k >= d_ff || cap < 0)
        return -1;
    const double z = oracle_threshold_z(k, d_ff);
    double *qd = (double *)malloc(sizeof(double) * (size_t)d_model);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < d_model; ++j)
            qd[j] = ld(q, qdtype, t * d_model + j);
        int64_t n = ffn_token(d_model, d_ff, r, z, wdtype, k1t, k2t, v, qd, y + t * d_model,
                              h ? h + t * d_ff : NULL, idx ? idx + t * cap : NULL, m ? m + t * cap : NULL, cap,
                              theta ? theta + t : NULL, mean ? mean + t : NULL, sd ? sd + t : NULL);
        if (counts) counts[t] = (int32_t)n;
    }
    free(qd);
    return 0;
}

/*
 * The same layer computed without exploiting its sparsity: the K2 dot and
 * the V row of EVERY neuron are used, the unselected neurons weighted by
 * GELU(max{h_i - theta, 0}) = GELU(0) = 0 (the "dense" cost the notes compare
 * the Spark FFN against).  Summed in ascending neuron order, the exact zeros
 * leave every sum unchanged, so y equals oracle_spark_ffn's bit for bit.
 * q [T][d_model] of dtype qdtype; y [T][d_model].
 */
int oracle_spark_ffn_dense(int64_t d_model, int64_t d_ff, int64_t r, int64_t k, int wdtype, const void *k1t,
                           const void *k2t, const void *v, int qdtype, const void *q, int64_t T, double *y)
{
    if (!k1t || !k2t || !v || !q || !y || T < 0 || r <= 0 || r >= d_model || k <= 0 || k >= d_ff)
        return -1;
    const double z = oracle_threshold_z(k, d_ff);
    const int64_t rc = d_model - r;
    double *qd = (double *)malloc(sizeof(double) * (size_t)d_model);
    double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *c = (double *)malloc(sizeof(double) * (size_t)d_ff);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < d_model; ++j)
            qd[j] = ld(q, qdtype, t * d_model + j);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < d_ff; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < r; ++j)
                s += ld(k1t, wdtype, i * r + j) * qd[j];
            h[i] = s;
        }
        double th;
        stat_topk_row(h, d_ff, z, NULL, NULL, &th, NULL, NULL, 0);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < d_ff; ++i) {
            double g = 0.0;
            for (int64_t j = 0; j < rc; ++j)
                g += ld(k2t, wdtype, i * rc + j) * qd[r + j];
            const double m = h[i] > th ? h[i] - th : 0.0;
            c[i] = oracle_gelu_tanh(m) * g;
        }
#pragma omp parallel for schedule(static)
        for (int64_t col = 0; col < d_model; ++col) {
            double s = 0.0;
            for (int64_t i = 0; i < d_ff; ++i)
                s += c[i] * ld(v, wdtype, i * d_model + col);
            y[t * d_model + col] = s;
        }
    }
    free(qd);
    free(h);
    free(c);
    return 0;
}

/*
 * A stack of n_layers independent Spark FFN layers applied in sequence to
 * each of T tokens: layer l+1 reads q_{l+1} = y_l / sqrt(mean(y_l^2) + eps)
 * (RMS normalisation with unit gain and no residual).  The returned y is the
 * last layer's output before normalisation.  k1t/k2t/v are arrays of
 * n_layers pointers.  Optional: counts [T][n_layers]; q_trace
 * [T][n_layers][d_model] receives each layer's input.
 */
int oracle_decode_stack(int64_t d_model, int64_t d_ff, int64_t r, int64_t k, int wdtype, int n_layers,
                        const void *const *k1t, const void *const *k2t, const void *const *v, const float *q0,
                        int64_t T, double eps, double *y, int32_t *counts, double *q_trace)
{
    if (!k1t || !k2t || !v || !q0 || !y || n_layers <= 0 || T < 0 || r <= 0 || r >= d_model || k <= 0 ||
        k >= d_ff)
        return -1;
    const double z = oracle_threshold_z(k, d_ff);
    double *q = (double *)malloc(sizeof(double) * (size_t)d_model);
    double *yl = (double *)malloc(sizeof(double) * (size_t)d_model);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < d_model; ++j)
            q[j] = (double)q0[t * d_model + j];
        for (int l = 0; l < n_layers; ++l) {
            if (q_trace)
                memcpy(q_trace + (t * n_layers + l) * d_model, q, sizeof(double) * (size_t)d_model);
            int64_t n = ffn_token(d_model, d_ff, r, z, wdtype, k1t[l], k2t[l], v[l], q, yl, NULL, NULL, NULL, 0,
                                  NULL, NULL, NULL);
            if (counts) counts[t * n_layers + l] = (int32_t)n;
            if (l + 1 < n_layers) {
                double ss = 0.0;
                for (int64_t j = 0; j < d_model; ++j)
                    ss += yl[j] * yl[j];
                double inv = 1.0 / sqrt(ss / (double)d_model + eps);
                for (int64_t j = 0; j < d_model; ++j)
                    q[j] = yl[j] * inv;
            }
        }
        memcpy(y + t * d_model, yl, sizeof(double) * (size_t)d_model);
    }
    free(q);
    free(yl);
    return 0;
}

/*
 * Spark attention for one query over the first n tokens of one KV head's
 * cache (rows j < n of a cache with N rows per head), the "Spark Attention"
 * item of the notes' key-design section: predictor scores s_j = q[:r].k1_j,
 * statistical top-k of s with k_attn (every token when n <= k_attn), softmax
 * of s over the selected set, softplus of q[r:].k2_j, and the weighted sum of
 * the v rows.  qi is the index of the query's first element in q.
 */
static void attn_query(int dtype, const void *q, int64_t qi, const void *k1, const void *k2, const void *v,
                       int64_t g, int64_t N, int64_t n, int64_t hd, int64_t r, int64_t k_attn, double *o,
                       int32_t *count, double *theta, double *scores)
{
    const int64_t rc = hd - r;
    const int dense = n <= k_attn;
    const double z = dense ? 0.0 : oracle_threshold_z(k_attn, n);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    int32_t *S = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    for (int64_t j = 0; j < n; ++j) {
        double a = 0.0;
        for (int64_t c = 0; c < r; ++c)
            a += ld(q, dtype, qi + c) * ld(k1, dtype, (g * N + j) * r + c);
        s[j] = a;
    }
    if (scores) memcpy(scores, s, sizeof(double) * (size_t)n);
    int64_t m;
    double th = NAN;
    if (dense) {
        for (int64_t j = 0; j < n; ++j)
            S[j] = (int32_t)j;
        m = n;
    } else {
        m = stat_topk_row(s, n, z, NULL, NULL, &th, S, NULL, n);
    }
    for (int64_t c = 0; c < hd; ++c)
        o[c] = 0.0;
    if (m > 0) {
        double smax = -INFINITY;
        for (int64_t t = 0; t < m; ++t)
            if (s[S[t]] > smax) smax = s[S[t]];
        double den = 0.0;
        for (int64_t t = 0; t < m; ++t)
            den += exp(s[S[t]] - smax);
        for (int64_t t = 0; t < m; ++t) {
            const int64_t j = S[t];
            double w = exp(s[j] - smax) / den;
            double a = 0.0;
            for (int64_t c = 0; c < rc; ++c)
                a += ld(q, dtype, qi + r + c) * ld(k2, dtype, (g * N + j) * rc + c);
            double wu = w * oracle_softplus(a);
            for (int64_t c = 0; c < hd; ++c)
                o[c] += wu * ld(v, dtype, (g * N + j) * hd + c);
        }
    }
    if (count) *count = (int32_t)m;
    if (theta) *theta = th;
    free(s);
    free(S);
}

/*
 * Spark attention, one decode step (notes, "Spark Attention" item).
 * q [Hq][hd]; k1 [Hkv][n_ctx][r] (predictor key dims); k2 [Hkv][n_ctx][hd-r]
 * (compute key dims); v [Hkv][n_ctx][hd]; all of dtype `dtype`.  Query head h
 * uses KV head h / (Hq/Hkv).  Per head: predictor scores s_j = q[:r].k1_j;
 * selected set S by statistical top-k with k_attn (all tokens when
 * n_ctx <= k_attn); weights w = softmax of s over S; gate u_j =
 * softplus(q[r:].k2_j); out[h] = sum_{j in S} w_j u_j v_j.
 * Optional: counts [Hq], theta [Hq] (NAN when all tokens are attended),
 * scores [Hq][n_ctx].
 */
int oracle_spark_attn_decode(int dtype, const void *q, const void *k1, const void *k2, const void *v, int64_t Hq,
                             int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double *out,
                             int32_t *counts, double *theta, double *scores)
{
    if (!q || !k1 || !k2 || !v || !out || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || n_ctx <= 0 || hd <= 0 ||
        r <= 0 || r >= hd || k_attn <= 0)
        return -1;
    const int64_t group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < Hq; ++h)
        attn_query(dtype, q, h * hd, k1, k2, v, h / group, n_ctx, n_ctx, hd, r, k_attn, out + h * hd,
                   counts ? counts + h : NULL, theta ? theta + h : NULL, scores ? scores + h * n_ctx : NULL);
    return 0;
}

/*
 * Spark attention over a whole prompt (causal prefill): the query of
 * position t attends over positions 0..t of the same cache, each query with
 * its own statistical top-k over its t + 1 scores ("Spark Attention" item;
 * the prefix reading is the causal form of the same operator).
 *   q [T][Hq][hd]; k1 [Hkv][T][r]; k2 [Hkv][T][hd-r]; v [Hkv][T][hd];
 *   out [T][Hq][hd]; counts, theta [T][Hq] (theta NaN when t + 1 <= k_attn).
 */
int oracle_spark_attn_prefill(int dtype, const void *q, const void *k1, const void *k2, const void *v, int64_t T,
                              int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, double *out,
                              int32_t *counts, double *theta)
{
    if (!q || !k1 || !k2 || !v || !out || T <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || hd <= 0 || r <= 0 ||
        r >= hd || k_attn <= 0)
        return -1;
    const int64_t group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t th = 0; th < T * Hq; ++th) {
        const int64_t t = th / Hq, h = th % Hq;
        attn_query(dtype, q, th * hd, k1, k2, v, h / group, T, t + 1, hd, r, k_attn, out + th * hd,
                   counts ? counts + th : NULL, theta ? theta + th : NULL, NULL);
    }
    return 0;
}
