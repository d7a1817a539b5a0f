// C ABI entry points (include/spark_ffn.h): argument checks, workspace sizing,
// threshold constant, dispatch to the gfx950 kernels.  Every check runs before
// the first device call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.hpp"
#include "spark_ffn.h"

namespace spark {

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace spark

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? SPARK_OK : SPARK_EHIP; }

int check_ffn_shape(const spark_ffn_shape* s) {
  if (!s) return SPARK_EINVAL;
  // The dtype field is read as the int it holds: a C caller or a foreign-function
  // layer may store any int there, and C++ may not load an out-of-range value
  // as the enum type itself.
  int wd = 0;
  static_assert(sizeof(wd) == sizeof(s->wdtype), "spark_dtype is int-sized");
  std::memcpy(&wd, &s->wdtype, sizeof wd);
  if (wd != SPARK_F32 && wd != SPARK_BF16) return SPARK_EUNSUPPORTED;
  if (s->d_model <= 0 || s->d_ff <= 0 || s->r <= 0 || s->r >= s->d_model) return SPARK_EINVAL;
  if (s->k <= 0 || s->k >= s->d_ff) return SPARK_EINVAL;
  const int64_t cn = s->wdtype == SPARK_BF16 ? 8 : 4;  // elements per 16-byte chunk
  if (s->r % cn != 0 || (s->d_model - s->r) % cn != 0) return SPARK_EINVAL;
  return SPARK_OK;
}

int check_weights(const spark_ffn_weights& w) {
  if (!w.k1t || !w.k2t || !w.v) return SPARK_EINVAL;
  if (!aligned(w.k1t, 16) || !aligned(w.k2t, 16) || !aligned(w.v, 16)) return SPARK_EINVAL;
  return SPARK_OK;
}

// Bytes at the start of a batched-decode workspace kept for the header of the
// single-token persistent kernel (exchange tags, failure mark and count).
constexpr size_t kBatchedHeader = 256;

int decode_limits(const spark_ffn_shape* s) {
  if (s->d_model > spark::kDecodeMaxDModel || s->d_ff > 65536) return SPARK_EUNSUPPORTED;
  const int grid = spark::decode_grid(s->d_ff);
  if (grid <= 0 || grid > 256) return SPARK_EUNSUPPORTED;
  if ((s->d_ff + grid - 1) / grid > spark::kDecodeMaxNeuronsPerWG) return SPARK_EUNSUPPORTED;
  // each workgroup owns at most two 16-byte chunks of a V row
  const int64_t cn = s->wdtype == SPARK_BF16 ? 8 : 4;
  if (s->d_model % cn != 0 || (s->d_model / cn + grid - 1) / grid > 2) return SPARK_EUNSUPPORTED;
  return SPARK_OK;
}

// Where a batched-decode workspace's layer-by-layer buffers start: after the
// whole layout of the single-token persistent kernel when the shape takes
// that kernel (a call with one token runs it), so that neither form's
// tagged exchange words ever share memory with the other's plain values and
// a stale value can never pass for a tag; else after the header alone.
size_t batched_offset(const spark_ffn_shape* s) {
  if (decode_limits(s) != SPARK_OK) return kBatchedHeader;
  const size_t d = spark::decode_workspace_bytes(s->d_model, s->d_ff, spark::kDecodeMaxLayersPerLaunch + 1, 1,
                                                 spark::decode_grid(s->d_ff));
  return std::max(kBatchedHeader, (d + 255) / 256 * 256);
}

}  // namespace

extern "C" {

const char* spark_status_string(int status) {
  switch (status) {
    case SPARK_OK: return "ok";
    case SPARK_EINVAL: return "invalid argument (size, k, null pointer, alignment or stride)";
    case SPARK_EUNSUPPORTED: return "unsupported dtype or size";
    case SPARK_EHIP: return "HIP runtime error while launching";
    case SPARK_EWORKSPACE: return "workspace missing, misaligned or too small";
    default: return "unknown status";
  }
}

int stat_topk(const float* x, int64_t rows, int64_t d, int64_t ldx, int64_t k, float* vals, int32_t* idx,
              int64_t cap, int32_t* counts, float* theta, hipStream_t stream) {
  if (rows < 0 || d <= 0 || ldx < d || k <= 0 || k >= d || cap < 0) return SPARK_EINVAL;
  if (d > 65536) return SPARK_EUNSUPPORTED;
  if (rows > 0 && (!x || !counts)) return SPARK_EINVAL;
  if (cap > 0 && rows > 0 && !vals && !idx) cap = 0;
  if (rows == 0) return SPARK_OK;
  const double z = spark_threshold_z(k, d);
  return hip_status(spark::launch_stat_topk(x, rows, d, ldx, z, vals, idx, cap, counts, theta, stream));
}

static int check_huber(const float* x, const void* other, const float* out, int64_t rows, int64_t d, int64_t k,
                       float delta) {
  if (rows < 0 || d <= 0 || k <= 0 || k >= d || !(delta > 0.f) || !std::isfinite(delta)) return SPARK_EINVAL;
  if (d > 65536) return SPARK_EUNSUPPORTED;
  if (rows > 0 && (!x || !other || !out)) return SPARK_EINVAL;
  return SPARK_OK;
}

int stat_topk_huber_forward(const float* x, int64_t rows, int64_t d, int64_t k, float delta, float* y, float* theta,
                            hipStream_t stream) {
  const int st = check_huber(x, y, y, rows, d, k, delta);
  if (st != SPARK_OK || rows == 0) return st;
  return hip_status(spark::launch_stat_topk_huber(false, x, nullptr, rows, d, spark_threshold_z(k, d), delta, y, theta,
                                                  stream));
}

int stat_topk_huber_backward(const float* x, const float* dy, int64_t rows, int64_t d, int64_t k, float delta,
                             float* dx, hipStream_t stream) {
  const int st = check_huber(x, dy, dx, rows, d, k, delta);
  if (st != SPARK_OK || rows == 0) return st;
  return hip_status(spark::launch_stat_topk_huber(true, x, dy, rows, d, spark_threshold_z(k, d), delta, dx, nullptr,
                                                  stream));
}

int64_t spark_ffn_decode_tags(int n_layers, int64_t T) {
  if (n_layers < 1 || T < 0) return -1;
  const int64_t launches = (n_layers + spark::kDecodeMaxLayersPerLaunch - 1) / spark::kDecodeMaxLayersPerLaunch;
  return T * (3 * (int64_t)n_layers - launches);
}

int spark_ffn_decode_workspace_size(const spark_ffn_shape* s, int n_layers, int64_t T, size_t* bytes) {
  if (!bytes) return SPARK_EINVAL;
  int st = check_ffn_shape(s);
  if (st != SPARK_OK) return st;
  if (n_layers < 1 || T < 0) return SPARK_EINVAL;
  st = decode_limits(s);
  if (st != SPARK_OK) return st;
  *bytes = spark::decode_workspace_bytes(s->d_model, s->d_ff, n_layers, T, spark::decode_grid(s->d_ff));
  return SPARK_OK;
}

int spark_ffn_decode(const spark_ffn_shape* s, const spark_ffn_weights* layers, int n_layers, const float* q,
                     int64_t T, float* y, float rms_eps, const spark_ffn_trace* trace, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_ffn_shape(s);
  if (st != SPARK_OK) return st;
  if (n_layers < 1 || !layers || T < 0 || !(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return SPARK_EINVAL;
  st = decode_limits(s);
  if (st != SPARK_OK) return st;
  if (T > 0 && (!q || !y)) return SPARK_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    st = check_weights(layers[l]);
    if (st != SPARK_OK) return st;
  }
  if (trace && trace->idx && trace->cap < 0) return SPARK_EINVAL;
  if ((int64_t)T * n_layers * 3 >= (int64_t)1 << 31) return SPARK_EUNSUPPORTED;
  size_t need = 0;
  spark_ffn_decode_workspace_size(s, n_layers, T, &need);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  if (T == 0) return SPARK_OK;
  const double z = spark_threshold_z(s->k, s->d_ff);
  return hip_status(spark::launch_decode(*s, layers, n_layers, q, T, y, rms_eps, z, trace, ws, stream));
}

int spark_ffn_decode_noalloc(const spark_ffn_shape* s, const spark_ffn_weights* layers, int n_layers,
                             const float* q, int64_t T, float* y, float rms_eps, const spark_ffn_trace* trace,
                             hipStream_t stream) {
  int st = check_ffn_shape(s);
  if (st != SPARK_OK) return st;
  if (n_layers < 1 || !layers || T < 0 || !(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return SPARK_EINVAL;
  st = decode_limits(s);
  if (st != SPARK_OK) return st;
  if (T > 0 && (!q || !y)) return SPARK_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    st = check_weights(layers[l]);
    if (st != SPARK_OK) return st;
  }
  if (trace && trace->idx && trace->cap < 0) return SPARK_EINVAL;
  if ((int64_t)T * n_layers * 3 >= (int64_t)1 << 31) return SPARK_EUNSUPPORTED;
  size_t need = 0;
  spark_ffn_decode_workspace_size(s, n_layers, T, &need);
  if (need > spark::kNoAllocScratchBytes) return SPARK_EUNSUPPORTED;  // beyond the built-in scratch
  if (T == 0) return SPARK_OK;
  const double z = spark_threshold_z(s->k, s->d_ff);
  return hip_status(spark::launch_decode_noalloc(*s, layers, n_layers, q, T, y, rms_eps, z, trace,
                                                 (uint64_t)spark_ffn_decode_tags(n_layers, T), stream));
}

size_t spark_ffn_decode_noalloc_max_bytes(void) { return spark::kNoAllocScratchBytes; }

int spark_ffn_decode_batched_workspace_size(const spark_ffn_shape* s, int64_t B, size_t* bytes) {
  if (!bytes) return SPARK_EINVAL;
  int st = check_ffn_shape(s);
  if (st != SPARK_OK) return st;
  if (B < 0) return SPARK_EINVAL;
  if (B > spark::kBatchMax || s->d_model > spark::kDecodeMaxDModel || s->d_ff > 65536) return SPARK_EUNSUPPORTED;
  const int64_t wide = s->r > s->d_model - s->r ? s->r : s->d_model - s->r;
  const int64_t slots = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;  // token slots of the kernels
  if (slots * wide * 4 > spark::kBatchMaxLds) return SPARK_EUNSUPPORTED;
  *bytes = batched_offset(s) + spark::decode_batched_workspace_bytes(s->d_model, s->d_ff, B > 0 ? B : 1);
  return SPARK_OK;
}

int spark_ffn_decode_batched(const spark_ffn_shape* s, const spark_ffn_weights* layers, int n_layers,
                             const float* q, int64_t B, float* y, float rms_eps, const spark_ffn_trace* trace,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  int st = spark_ffn_decode_batched_workspace_size(s, B, &need);
  if (st != SPARK_OK) return st;
  if (n_layers < 1 || !layers || !(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return SPARK_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    st = check_weights(layers[l]);
    if (st != SPARK_OK) return st;
  }
  if (B > 0 && (!q || !y || !aligned(q, 16) || !aligned(y, 16))) return SPARK_EINVAL;
  if (trace && trace->idx && trace->cap < 0) return SPARK_EINVAL;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  if ((int64_t)n_layers * 3 >= (int64_t)1 << 31) return SPARK_EUNSUPPORTED;
  if (B == 0) return SPARK_OK;
  const double z = spark_threshold_z(s->k, s->d_ff);
  // one token: the single-token persistent kernel; more: the layer-by-layer
  // kernels (the header's tags and failure record shared with it)
  if (B == 1 && decode_limits(s) == SPARK_OK)
    return hip_status(spark::launch_decode(*s, layers, n_layers, q, 1, y, rms_eps, z, trace, ws, stream));
  return hip_status(spark::launch_decode_batched(*s, layers, n_layers, q, B, y, rms_eps, z, trace,
                                                 (char*)ws + batched_offset(s), (uint64_t*)ws, stream));
}

int spark_ffn_prefill_workspace_size(const spark_ffn_shape* s, int64_t T, size_t* bytes) {
  if (!bytes) return SPARK_EINVAL;
  int st = check_ffn_shape(s);
  if (st != SPARK_OK) return st;
  if (T < 0) return SPARK_EINVAL;
  if (s->wdtype != SPARK_BF16 || s->d_ff % 256 != 0 || s->r % 64 != 0 || s->d_model % 8 != 0 ||
      s->d_model > 8192 || s->d_ff > 65536)
    return SPARK_EUNSUPPORTED;
  *bytes = spark::prefill_workspace_bytes(s->d_model, s->d_ff, T);
  return SPARK_OK;
}

int spark_ffn_prefill(const spark_ffn_shape* s, const spark_ffn_weights* w, const void* Q, int64_t T, float* Y,
                      const spark_ffn_trace* trace, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  int st = spark_ffn_prefill_workspace_size(s, T, &need);
  if (st != SPARK_OK) return st;
  if (!w) return SPARK_EINVAL;
  st = check_weights(*w);
  if (st != SPARK_OK) return st;
  if (T > 0 && (!Q || !Y || !aligned(Q, 16))) return SPARK_EINVAL;
  if (trace && trace->idx && trace->cap < 0) return SPARK_EINVAL;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  if (T == 0) return SPARK_OK;
  const double z = spark_threshold_z(s->k, s->d_ff);
  return hip_status(spark::launch_prefill(*s, *w, Q, T, Y, z, trace, ws, stream));
}

int spark_ffn_prefill_gathered_workspace_size(const spark_ffn_shape* s, int64_t T, size_t* bytes) {
  size_t dense = 0;
  const int st = spark_ffn_prefill_workspace_size(s, T, &dense);  // the same shape limits
  if (st != SPARK_OK) return st;
  *bytes = spark::prefill_gathered_workspace_bytes(s->d_model, s->d_ff, T);
  return SPARK_OK;
}

int spark_ffn_prefill_gathered(const spark_ffn_shape* s, const spark_ffn_weights* w, const void* Q, int64_t T,
                               float* Y, const spark_ffn_trace* trace, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  int st = spark_ffn_prefill_gathered_workspace_size(s, T, &need);
  if (st != SPARK_OK) return st;
  if (!w) return SPARK_EINVAL;
  st = check_weights(*w);
  if (st != SPARK_OK) return st;
  if (T > 0 && (!Q || !Y || !aligned(Q, 16) || !aligned(Y, 16))) return SPARK_EINVAL;
  if (trace && trace->idx && trace->cap < 0) return SPARK_EINVAL;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  if (T == 0) return SPARK_OK;
  const double z = spark_threshold_z(s->k, s->d_ff);
  return hip_status(spark::launch_prefill_gathered(*s, *w, Q, T, Y, z, trace, ws, stream));
}

int spark_ffn_prefill_scores(const spark_ffn_shape* s, const spark_ffn_weights* w, const void* Q, int64_t T, float* H,
                             hipStream_t stream) {
  size_t need = 0;
  const int st = spark_ffn_prefill_workspace_size(s, T, &need);  // the same shape limits as the whole prefill
  if (st != SPARK_OK) return st;
  if (!w) return SPARK_EINVAL;
  const int sw = check_weights(*w);
  if (sw != SPARK_OK) return sw;
  if (T > 0 && (!Q || !H || !aligned(Q, 16))) return SPARK_EINVAL;
  if (T == 0) return SPARK_OK;
  return hip_status(spark::launch_prefill_scores(*s, *w, Q, T, H, stream));
}

int spark_hbm_read_probe(const void* p, size_t bytes, float* sink, hipStream_t stream) {
  if (!p || !sink || bytes % 16 != 0 || !aligned(p, 16)) return SPARK_EINVAL;
  if (bytes == 0) return SPARK_OK;
  return hip_status(spark::launch_hbm_read_probe(p, bytes, sink, stream));
}

int spark_attn_workspace_size(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn,
                              size_t* bytes) {
  if (!bytes) return SPARK_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || hd <= 0 || r <= 0 || r >= hd || n_ctx <= 0 || k_attn <= 0)
    return SPARK_EINVAL;
  if (r % 8 != 0 || (hd - r) % 8 != 0) return SPARK_EINVAL;
  if (hd > 512 || n_ctx > (1 << 20) || Hq > 1024) return SPARK_EUNSUPPORTED;
  *bytes = spark::attn_workspace_bytes(Hq, Hkv, n_ctx, hd, r, k_attn);
  return SPARK_OK;
}

int spark_attn_decode(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq, int64_t Hkv,
                      int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, float* out, int32_t* counts,
                      int32_t* idx, int64_t cap, float* theta, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  int st = spark_attn_workspace_size(Hq, Hkv, n_ctx, hd, r, k_attn, &need);
  if (st != SPARK_OK) return st;
  if (!q || !k1 || !k2 || !v || !out) return SPARK_EINVAL;
  if (!aligned(q, 16) || !aligned(k1, 16) || !aligned(k2, 16) || !aligned(v, 16)) return SPARK_EINVAL;
  if (idx && cap < 0) return SPARK_EINVAL;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  const double z = n_ctx <= k_attn ? 0.0 : spark_threshold_z(k_attn, n_ctx);
  return hip_status(spark::launch_attn_decode(q, k1, k2, v, Hq, Hkv, n_ctx, hd, r, k_attn, z, out, counts, idx,
                                              idx ? cap : 0, theta, ws, stream));
}

int spark_attn_prefill_workspace_size(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn,
                                      int64_t cap, size_t* bytes) {
  if (!bytes) return SPARK_EINVAL;
  if (T <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || hd <= 0 || r <= 0 || r >= hd || k_attn <= 0 || cap < 0)
    return SPARK_EINVAL;
  if (r % 8 != 0 || (hd - r) % 8 != 0) return SPARK_EINVAL;
  if (hd > 512 || T > 16384 || Hq > 1024) return SPARK_EUNSUPPORTED;
  *bytes = spark::attn_prefill_workspace_bytes(T, Hq, Hkv, hd, r, cap > 0);
  return SPARK_OK;
}

int spark_attn_prefill(const void* q, const void* k1, const void* k2, const void* v, int64_t T, int64_t Hq,
                       int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out, int32_t* counts, int32_t* idx,
                       int64_t cap, float* theta, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (idx && cap < 0) return SPARK_EINVAL;
  const int64_t lcap = idx ? cap : 0;
  size_t need = 0;
  int st = spark_attn_prefill_workspace_size(T, Hq, Hkv, hd, r, k_attn, lcap, &need);
  if (st != SPARK_OK) return st;
  if (!q || !k1 || !k2 || !v || !out) return SPARK_EINVAL;
  if (!aligned(q, 16) || !aligned(k1, 16) || !aligned(k2, 16) || !aligned(v, 16)) return SPARK_EINVAL;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPARK_EWORKSPACE;
  return hip_status(spark::launch_attn_prefill(q, k1, k2, v, T, Hq, Hkv, hd, r, k_attn, out, counts,
                                               lcap > 0 ? idx : nullptr, lcap, theta, ws, stream));
}

}  // extern "C"
