/*
 * spark_ffn.h -- C ABI of the MI355X (gfx950) Spark FFN library.
 *
 * The operations are those of the Spark Transformer (arXiv 2506.06644,
 * "Spark Transformer: Reactivating Sparsity in FFN and Attention"); the
 * statements of the method used here are in the reading notes of that paper,
 * section "方法详解 / 关键设计" (method / key design), items "Spark FFN",
 * "Spark Attention" and "Statistical Top-k".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory.  Every array argument is a DEVICE pointer (memory of the current
 *    HIP device), except the shape/weight/trace structs themselves and the
 *    `layers` array of spark_ffn_decode, which live in host memory.  The caller
 *    owns all memory; the library never allocates or frees device memory.
 *    Scratch memory is the caller's workspace `ws` of `ws_bytes` bytes, sized
 *    with the matching *_workspace_size function (256-byte aligned base).
 *  - Layout.  Row-major and contiguous.  Weights of one Spark FFN layer:
 *      k1t [d_ff][r]          K1 transposed: row i is neuron i's predictor key
 *      k2t [d_ff][d_model-r]  K2 transposed: row i is neuron i's compute key
 *      v   [d_ff][d_model]    row i is neuron i's value row
 *    Spark attention KV cache, split along the key dimension:
 *      k1 [Hkv][n_ctx][r], k2 [Hkv][n_ctx][hd-r], v [Hkv][n_ctx][hd].
 *  - Streams.  Work is enqueued on `stream` (NULL = the default stream) and
 *    runs asynchronously; nothing synchronises the host.
 *  - Errors.  Return SPARK_OK or a negative status.  All argument checks run
 *    before the first device call, so a non-OK status means nothing was
 *    enqueued -- except SPARK_EHIP, returned when the HIP runtime rejects a
 *    launch (the error is the one hipGetLastError reported).  No C++
 *    exception crosses this interface.  spark_status_string() names a status.
 *  - Capacity.  Per-row index/value lists have `cap` slots.  `counts` always
 *    receives the TRUE number of selected entries; when it exceeds `cap` only
 *    the first `cap` (lowest indices) are stored.  cap = d never truncates.
 *  - Determinism.  Every reduction runs in a fixed order: identical inputs
 *    give bit-identical outputs.
 */
#ifndef SPARK_FFN_H
#define SPARK_FFN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SPARK_OK = 0,
    SPARK_EINVAL = -1,       /* bad size, k, pointer, alignment or stride */
    SPARK_EUNSUPPORTED = -2, /* a dtype or size outside what is built */
    SPARK_EHIP = -3,         /* the HIP runtime failed a launch */
    SPARK_EWORKSPACE = -4    /* ws is NULL, misaligned or smaller than required */
};

typedef enum { SPARK_F32 = 0, SPARK_BF16 = 1 } spark_dtype;

/* One Spark FFN layer shape.  0 < r < d_model (q[:r] feeds the predictor,
 * q[r:] the compute keys); 0 < k < d_ff (target number of active neurons). */
typedef struct {
    int64_t d_model, d_ff, r, k;
    spark_dtype wdtype; /* dtype of k1t, k2t and v */
} spark_ffn_shape;

/* Device pointers to one layer's weights (layouts above). */
typedef struct {
    const void *k1t, *k2t, *v;
} spark_ffn_weights;

/* Optional per-layer outputs for inspection; every pointer may be NULL.
 * For spark_ffn_prefill n_layers is 1. */
typedef struct {
    int32_t *counts; /* [T][n_layers] true number of selected neurons */
    int32_t *idx;    /* [T][n_layers][cap] selected neurons, ascending */
    float *theta;    /* [T][n_layers] threshold used */
    float *q_in;     /* [T][n_layers][d_model] each layer's input q (decode only) */
    int64_t cap;     /* slots per (token, layer) in idx */
} spark_ffn_trace;

/*
 * Statistical top-k ("Statistical Top-k" item): for each of `rows` fp32 rows
 * x[row*ldx + 0..d), theta = mean + std * Q(1 - k/d) with the population std
 * (1/d) and Q the standard-normal quantile; the selected set is
 * {i : x_i > theta} in ascending order, and the soft-threshold value of a
 * selected entry is x_i - theta (the operator max{x - theta, 0} restricted to
 * its nonzeros).
 *   vals [rows][cap] fp32, idx [rows][cap] int32: first min(count, cap)
 *       entries of each row (both may be NULL; then nothing is listed);
 *   counts [rows] int32 (required);  theta [rows] fp32 (may be NULL).
 * Requires 0 < k < d <= 65536, ldx >= d, rows >= 0, cap >= 0.  No workspace.
 * Rows with zero spread select nothing.
 */
int stat_topk(const float *x, int64_t rows, int64_t d, int64_t ldx, int64_t k, float *vals, int32_t *idx,
              int64_t cap, int32_t *counts, float *theta, hipStream_t stream);

/*
 * Training side of the statistical top-k ("Statistical Top-k" item: with
 * Huber smoothing the operator is continuously differentiable).  The smoothing
 * taken: the soft-threshold max{u, 0}, u = x - theta, becomes
 *     h(u) = 0 (u <= 0),  u^2 / (2 delta) (0 < u < delta),  u - delta/2 (u >= delta),
 * with theta = mean + std * Q(1 - k/d) (population std) as above.
 *   forward:  y [rows][d] = h(x - theta) for every entry (dense; zero at and
 *             below theta); theta [rows] may be NULL.
 *   backward: dx [rows][d] = dL/dx given dy = dL/dy [rows][d], through theta's
 *             dependence on the row:  a_i = dy_i h'(x_i - theta),
 *             A = sum_i a_i,  dx_j = a_j - (A/d) (1 + Q(1 - k/d) (x_j - mean)/std);
 *             a row with zero spread gets dx = 0.  x is the forward's input.
 * All arrays fp32 and contiguous (row stride d); any alignment.  Requires
 * 0 < k < d <= 65536, delta > 0 finite, rows >= 0.  No workspace.
 */
int stat_topk_huber_forward(const float *x, int64_t rows, int64_t d, int64_t k, float delta, float *y, float *theta,
                            hipStream_t stream);
int stat_topk_huber_backward(const float *x, const float *dy, int64_t rows, int64_t d, int64_t k, float delta,
                             float *dx, hipStream_t stream);

/*
 * Spark FFN decode ("Spark FFN" item): for each of T independent tokens, run
 * the stack of n_layers Spark FFN layers
 *     y_l = V (GELU(StatTopk(K1^T q_l[:r])) (.) (K2^T q_l[r:]))
 * where StatTopk is the statistical top-k above with k = s->k over the d_ff
 * predictor scores, GELU is the tanh form, and only the selected K2 columns
 * (k2t rows) and V rows are read.  Between layers
 *     q_{l+1} = y_l / sqrt(mean(y_l^2) + rms_eps)      (unit gain, no residual).
 *   q [T][d_model] fp32 input of layer 0;  y [T][d_model] fp32 output of the
 *   last layer (before normalisation);  layers: host array of n_layers weight
 *   sets; trace may be NULL.
 * Weights fp32 or bf16; arithmetic fp32 with fp32 accumulation.
 * Requires d_model <= 8192, d_ff <= 65536, 1 <= n_layers, T >= 0, rms_eps >= 0,
 * k1t, k2t and v base pointers 16-byte aligned, and r and d_model - r
 * multiples of 8 elements (bf16) or 4 elements (fp32), so that every weight
 * row is whole 16-byte chunks; SPARK_EINVAL otherwise.
 * The kernel is one persistent grid of one workgroup per compute unit whose
 * workgroups exchange data while they run, so the device must hold the whole
 * grid at once: SPARK_EHIP if it cannot.  Other work running on the device
 * at the same time can delay workgroups; a call whose waits then time out
 * fails as described below (it does not hang).
 * Workspace: zero-filled before its first use, then kept between calls: it
 * carries the 32-bit tags of the grid-wide exchanges from call to call, and a
 * call uses spark_ffn_decode_tags(n_layers, T) of them.  Zero the workspace
 * again before the tags used since it was last zeroed would exceed
 * 2^32 - 1 (a tag must never repeat while a word carrying it can still be
 * read).  Calls that overlap on one workspace race.
 * Failure: every exchange wait is bounded.  When one times out (a grid that
 * could not make progress), the call ends early, the columns of y it did not
 * finish read NaN, and the 8-byte counter at byte offset 16 of the workspace
 * is incremented (once per failed call); the tags still advance as after a
 * complete call, so the next call on the workspace is unaffected.  The
 * 8-byte word at byte offset 24 is a test hook that drives this failure
 * path from the host: when nonzero, every wait is bounded by that many
 * polling rounds and the first exchange cannot complete, so the call fails;
 * leave it zero.
 */
int spark_ffn_decode(const spark_ffn_shape *s, const spark_ffn_weights *layers, int n_layers, const float *q,
                     int64_t T, float *y, float rms_eps, const spark_ffn_trace *trace, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * spark_ffn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and failure behaviour as spark_ffn_decode, without
 * the workspace: the exchanges use a scratch array built into the library,
 * one per device, of spark_ffn_decode_noalloc_max_bytes() bytes (2 MiB),
 * which each device holds until the process ends.  This entry point makes no
 * allocation (no hipMalloc, hipFree or allocating library call).
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress, with the device current) and clears it with a
 *     small kernel on `stream`; it is cleared the same way whenever the
 *     exchange tags used since the last clear would pass 2^32 - 1.
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's contents: calls that overlap on one device (other streams, other
 *     host threads) race, so serialise them.
 *   - Sizes whose spark_ffn_decode_workspace_size exceeds the array return
 *     SPARK_EUNSUPPORTED before anything is enqueued (every shape of up to 32
 *     layers fits; more layers need 8 * T * d_model bytes more).
 */
int spark_ffn_decode_noalloc(const spark_ffn_shape *s, const spark_ffn_weights *layers, int n_layers,
                             const float *q, int64_t T, float *y, float rms_eps, const spark_ffn_trace *trace,
                             hipStream_t stream);

/* Bytes of the per-device scratch array spark_ffn_decode_noalloc uses. */
size_t spark_ffn_decode_noalloc_max_bytes(void);

/* Exchange tags one spark_ffn_decode call with these arguments uses: T times
 * (3 n_layers - the number of launches), a launch holding up to 32 layers.
 * Returns -1 for n_layers < 1 or T < 0. */
int64_t spark_ffn_decode_tags(int n_layers, int64_t T);

/*
 * Batched Spark FFN decode: the computation of spark_ffn_decode for B
 * independent tokens (q [B][d_model] fp32 in, y [B][d_model] fp32 out, the
 * same trace layout with T = B), with the batch processed layer by layer: one
 * read of K1 per layer serves all B tokens, and the K2 and V rows of a neuron
 * are read once for all the tokens that select it (the union of the
 * per-token selected sets).  The method is that of spark_ffn_decode (reading
 * notes of the Spark Transformer, section "方法详解 / 关键设计", items "Spark
 * FFN" and "Statistical Top-k"); results equal spark_ffn_decode's up to the
 * order of fp32 sums.
 * Forms, chosen per call: B = 1 (within spark_ffn_decode's limits) runs the
 * single-token persistent kernel; larger batches run per layer one kernel for
 * the predictor and the gate, whose workgroups exchange the score statistics
 * while they run (bf16 weights, r and d_model - r multiples of 32 and at most
 * 1280, d_ff at most 256 x 40, and a grid the device holds at once), else a
 * predictor kernel and a gate kernel; then the V product (plus one kernel
 * when a trace is asked for).  After the exchanging kernel the V product sums
 * its slices itself, through tagged words in the workspace under the same
 * layer tag; otherwise one more kernel sums them.
 * Requires 0 <= B <= 8, d_model <= 8192, d_ff <= 65536,
 * P * max(r, d_model - r) * 4 <= 65536 with P = B rounded up to a power of
 * two, q and y 16-byte aligned, and the weight conditions of
 * spark_ffn_decode.  The workspace (spark_ffn_decode_batched_workspace_size,
 * 256-byte aligned, at least 256 bytes) must be zero-filled before its first
 * use and then handed unchanged to later calls: like spark_ffn_decode's it
 * carries the exchange tags (one call uses spark_ffn_decode_tags(n_layers, 1)
 * of them or fewer; zero it again before 2^32 - 1 are used) and the failure
 * record at byte offsets 16 (failed calls) and 24 (test hook, keep 0), both
 * used by the forms that exchange data while they run: a call whose exchange
 * wait times out (a grid the device could not keep running) returns SPARK_OK
 * with NaN in y and counts itself once at offset 16.  Calls that overlap on
 * one workspace race.
 */
int spark_ffn_decode_batched(const spark_ffn_shape *s, const spark_ffn_weights *layers, int n_layers,
                             const float *q, int64_t B, float *y, float rms_eps, const spark_ffn_trace *trace,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Spark FFN prefill: the same layer (one layer) applied to T tokens at once
 * (same result as spark_ffn_decode of one layer per token, without the
 * normalisation).  The predictor scores K1^T Q[:, :r] are a dense GEMM on the
 * matrix cores (fp32 scores), the statistical top-k runs per token over them,
 * and the gated K2 and V products run dense on the matrix cores with the
 * unselected neurons' gated values set to exact zeros.
 *   Q [T][d_model] of dtype s->wdtype; Y [T][d_model] fp32; trace may be NULL
 *   (its q_in is ignored).
 * Requires bf16 weights and Q, d_ff a multiple of 256, r a multiple of 64,
 * d_model a multiple of 8, d_model <= 8192, d_ff <= 65536.  The workspace
 * holds the scores, the gated values, a transposed copy of V and the K-split
 * partial sums of the output (added in a fixed order).
 */
int spark_ffn_prefill(const spark_ffn_shape *s, const spark_ffn_weights *w, const void *Q, int64_t T, float *Y,
                      const spark_ffn_trace *trace, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * spark_ffn_prefill with the K2 and V steps exactly as the "Spark FFN" item
 * states them: after the same dense predictor product and statistical top-k,
 * each token reads only its selected neurons' K2 rows (k2t) and V rows, the
 * gated values in fp32 and the V rows summed in ascending neuron order.
 * The same arguments, requirements and results as spark_ffn_prefill (up to
 * the rounding of the gated values, which that call feeds to the matrix
 * cores as bf16); Y must also be 16-byte aligned.  With i.i.d. selections the
 * dense products on the matrix cores are faster (each token's rows are
 * gathered from memory separately); this is the gathered form for
 * comparison and for selections that are sparser or clustered.  The
 * workspace (spark_ffn_prefill_gathered_workspace_size) holds the scores and
 * every token's full list: about 12 T d_ff bytes.
 */
int spark_ffn_prefill_gathered(const spark_ffn_shape *s, const spark_ffn_weights *w, const void *Q, int64_t T,
                               float *Y, const spark_ffn_trace *trace, void *ws, size_t ws_bytes,
                               hipStream_t stream);
int spark_ffn_prefill_gathered_workspace_size(const spark_ffn_shape *s, int64_t T, size_t *bytes);

/*
 * The predictor step of spark_ffn_prefill alone: H [T][d_ff] fp32 =
 * Q[:, :r] K1 (H[t][i] = q_t[:r] . k1t[i]), the dense bf16 product on the
 * matrix cores.  Same shape and weight requirements as spark_ffn_prefill; no
 * workspace.  (H is the input spark_ffn_prefill's statistical top-k reads.)
 */
int spark_ffn_prefill_scores(const spark_ffn_shape *s, const spark_ffn_weights *w, const void *Q, int64_t T, float *H,
                             hipStream_t stream);

/*
 * Measurement helper, not part of the method: streams `bytes` bytes (a
 * multiple of 16, 16-byte aligned base) from device memory p with 16-byte
 * nontemporal loads across the whole device and discards them (sink, one
 * float, is written only for a bit pattern no finite data produces).  Its
 * rate is the HBM read ceiling the decode kernel's bandwidth is compared to.
 */
int spark_hbm_read_probe(const void *p, size_t bytes, float *sink, hipStream_t stream);

/*
 * Spark attention decode ("Spark Attention" item): attention in the form of
 * the Spark FFN, with the key dimension split into a predictor part (first r
 * dims) and a compute part (last hd - r dims), sigma1 = softmax and
 * sigma2 = softplus.  For query head h (KV head g = h / (Hq/Hkv)):
 *     s_j = q_h[:r] . k1[g][j]                    (predictor scores, j < n_ctx)
 *     S   = statistical top-k of s with k_attn    (all j when n_ctx <= k_attn)
 *     w_j = softmax of s over S (unselected tokens get weight 0)
 *     u_j = softplus(q_h[r:] . k2[g][j])
 *     out_h = sum_{j in S} w_j u_j v[g][j]
 * No 1/sqrt(hd) factor is applied (scale q or k beforehand).
 *   q [Hq][hd] bf16; k1/k2/v bf16 as above; out [Hq][hd] fp32;
 *   counts [Hq] (may be NULL), idx [Hq][cap] (may be NULL), theta [Hq] (may be
 *   NULL; NaN when all tokens are attended).
 * Requires Hq % Hkv == 0, hd <= 512, 0 < r < hd, r and hd - r multiples of 8,
 * 1 <= n_ctx <= 1048576, k_attn >= 1.
 * Three launches on `stream` (scores and chunk statistics; per chunk the
 * selection, gates and a split-softmax partial; the merge).  The workspace
 * needs no initialisation.
 */
int spark_attn_decode(const void *q, const void *k1, const void *k2, const void *v, int64_t Hq, int64_t Hkv,
                      int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, float *out, int32_t *counts,
                      int32_t *idx, int64_t cap, float *theta, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Spark attention over a whole prompt, causal prefill ("Spark Attention"
 * item, in causal form): the query of position t attends over positions
 * 0..t of the same cache with its own statistical top-k over its t + 1
 * predictor scores (every position while t + 1 <= k_attn), softmax over the
 * selected set and softplus gates, as spark_attn_decode does for one query.
 *   q [T][Hq][hd] bf16 (position-major); k1 [Hkv][T][r], k2 [Hkv][T][hd-r],
 *   v [Hkv][T][hd] bf16; out [T][Hq][hd] fp32; counts [T][Hq] (may be NULL);
 *   idx [T][Hq][cap] int32 (may be NULL): the attended positions of each
 *   (t, h) in ascending order, the first min(count, cap) of them, the rest of
 *   the row's slots -1 (cap >= 0; with cap > 0 the workspace must be sized
 *   for that cap, since it then also holds a selection bitmask of
 *   T * Hq * ceil(T/32) words);
 *   theta [T][Hq] (may be NULL; NaN where t + 1 <= k_attn).
 * All products run on the matrix cores.  With r = hd - r in {32, 64, 128}
 * two fused kernels walk the keys of each query twice (moments and maximum
 * of the scores, then the gated weights and their product with V) and the
 * workspace holds V^T, two floats per (head, position) and the threshold
 * table; other head splits materialise Hq * T * T fp32 scores and bf16
 * weights in the workspace (unselected positions contribute exact zeros).
 * spark_attn_prefill_workspace_size gives the size for either.
 * Requires Hq % Hkv == 0, hd <= 512 and a multiple of 8, 0 < r < hd with r and
 * hd - r multiples of 8, 1 <= T <= 16384, k_attn >= 1.
 */
int spark_attn_prefill(const void *q, const void *k1, const void *k2, const void *v, int64_t T, int64_t Hq,
                       int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float *out, int32_t *counts, int32_t *idx,
                       int64_t cap, float *theta, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace sizes (bytes) for the calls above with the same arguments, on the
 * current device: some depend on its compute-unit count, and every call checks
 * ws_bytes against the size for the device current when it is made.  For
 * spark_attn_prefill, cap is the list capacity the call will pass with a
 * non-NULL idx (0 when it passes no list). */
int spark_ffn_decode_workspace_size(const spark_ffn_shape *s, int n_layers, int64_t T, size_t *bytes);
int spark_ffn_decode_batched_workspace_size(const spark_ffn_shape *s, int64_t B, size_t *bytes);
int spark_ffn_prefill_workspace_size(const spark_ffn_shape *s, int64_t T, size_t *bytes);
int spark_attn_workspace_size(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn,
                              size_t *bytes);
int spark_attn_prefill_workspace_size(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn,
                                      int64_t cap, size_t *bytes);

/* z = Q(1 - k/d), the standard-normal quantile the threshold uses (host fp64). */
double spark_threshold_z(int64_t k, int64_t d);

/* Text for a status code. */
const char *spark_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARK_FFN_H */
