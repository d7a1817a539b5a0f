// Host-only build of the C ABI layer (api.cpp, quantile.cpp) for the
// address and undefined-behaviour sanitizers.  The device side is replaced by
// stubs: the launchers record their arguments and return success, the
// workspace sizes are simple functions of the shape, and the two HIP runtime
// queries api.cpp makes report device 0 with 256 compute units.  The driver
// checks the status every entry point returns for valid and invalid
// arguments and that a valid call reaches its launcher once.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "internal.hpp"
#include "spark_ffn.h"

extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}

static int launches = 0;

namespace spark {
hipError_t launch_stat_topk(const float*, int64_t, int64_t, int64_t, double z, float*, int32_t*, int64_t, int32_t*,
                            float*, hipStream_t, const float*) {
  ++launches;
  return std::isfinite(z) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_stat_topk_huber(bool, const float*, const float*, int64_t, int64_t, double z, float delta, float*,
                                  float*, hipStream_t) {
  ++launches;
  return std::isfinite(z) && delta > 0.f ? hipSuccess : hipErrorInvalidValue;
}
size_t decode_workspace_bytes(int64_t d_model, int64_t, int n_layers, int64_t T, int grid) {
  return 4096 + (size_t)grid * 64 + (size_t)d_model * 64 + (n_layers > kDecodeMaxLayersPerLaunch ? 8 * T * d_model : 0);
}
int decode_grid(int64_t d_ff) { return (int)(d_ff < device_cu_count() ? d_ff : device_cu_count()); }
hipError_t launch_decode(const spark_ffn_shape&, const spark_ffn_weights*, int, const float*, int64_t, float*, float,
                         double z, const spark_ffn_trace*, void*, hipStream_t) {
  ++launches;
  return std::isfinite(z) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_decode_noalloc(const spark_ffn_shape&, const spark_ffn_weights*, int, const float*, int64_t,
                                 float*, float, double z, const spark_ffn_trace*, uint64_t tags, hipStream_t) {
  ++launches;
  return std::isfinite(z) && tags > 0 ? hipSuccess : hipErrorInvalidValue;
}
size_t decode_batched_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t B) {
  return (size_t)(d_model + d_ff) * B * 8;
}
hipError_t launch_decode_batched(const spark_ffn_shape&, const spark_ffn_weights*, int, const float*, int64_t, float*,
                                 float, double, const spark_ffn_trace*, void*, uint64_t*, hipStream_t) {
  ++launches;
  return hipSuccess;
}
size_t prefill_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T) { return (size_t)(d_model + d_ff) * T * 8; }
hipError_t launch_prefill(const spark_ffn_shape&, const spark_ffn_weights&, const void*, int64_t, float*, double,
                          const spark_ffn_trace*, void*, hipStream_t) {
  ++launches;
  return hipSuccess;
}
size_t prefill_gathered_workspace_bytes(int64_t, int64_t d_ff, int64_t T) { return (size_t)d_ff * T * 12 + 4096; }
hipError_t launch_prefill_gathered(const spark_ffn_shape&, const spark_ffn_weights&, const void*, int64_t, float*,
                                   double, const spark_ffn_trace*, void*, hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t launch_prefill_scores(const spark_ffn_shape&, const spark_ffn_weights&, const void*, int64_t, float*,
                                 hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t launch_hbm_read_probe(const void*, size_t bytes, float*, hipStream_t) {
  ++launches;
  return bytes % 16 == 0 ? hipSuccess : hipErrorInvalidValue;
}
size_t attn_workspace_bytes(int64_t Hq, int64_t, int64_t n_ctx, int64_t hd, int64_t, int64_t) {
  return (size_t)Hq * (n_ctx + hd) * 8;
}
size_t attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t, int64_t hd, int64_t, bool lists) {
  return (size_t)Hq * T * hd * 2 + (lists ? (size_t)T * Hq * ((T + 31) / 32) * 4 : 0);
}
hipError_t launch_attn_prefill(const void*, const void*, const void*, const void*, int64_t, int64_t, int64_t, int64_t,
                               int64_t, int64_t, float*, int32_t*, int32_t*, int64_t, float*, void*, hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t launch_attn_decode(const void*, const void*, const void*, const void*, int64_t, int64_t, int64_t, int64_t,
                              int64_t, int64_t, double, float*, int32_t*, int32_t*, int64_t, float*, void*,
                              hipStream_t) {
  ++launches;
  return hipSuccess;
}
}  // namespace spark

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  // fake, suitably aligned device addresses: the stubs never dereference them
  char* const P = (char*)(uintptr_t)(1 << 20);
  const float* x = (const float*)P;
  void* ws = P + (1 << 16);
  int32_t* counts = (int32_t*)(P + 4096);

  // threshold constant
  EXPECT(std::fabs(spark_threshold_z(737, 9216) - 1.405275953118082) < 1e-12);
  EXPECT(spark_threshold_z(5000, 10000) == 0.0);
  EXPECT(std::isnan(spark_threshold_z(0, 10)) && std::isnan(spark_threshold_z(10, 10)));
  for (int64_t d : {2, 3, 7, 1024, 9216, 65536, 1 << 20})
    for (int64_t k = 1; k < d; k += (d > 64 ? d / 37 + 1 : 1)) EXPECT(std::isfinite(spark_threshold_z(k, d)));

  // statistical top-k
  int n0 = launches;
  EXPECT(stat_topk(x, 16, 9216, 9216, 737, (float*)P, counts, 100, counts, nullptr, nullptr) == SPARK_OK);
  EXPECT(launches == n0 + 1);
  EXPECT(stat_topk(x, -1, 10, 10, 3, nullptr, nullptr, 0, counts, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk(x, 4, 10, 9, 3, nullptr, nullptr, 0, counts, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk(x, 4, 10, 10, 10, nullptr, nullptr, 0, counts, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk(x, 4, 70000, 70000, 3, nullptr, nullptr, 0, counts, nullptr, nullptr) == SPARK_EUNSUPPORTED);
  EXPECT(stat_topk(nullptr, 0, 10, 10, 3, nullptr, nullptr, 0, nullptr, nullptr, nullptr) == SPARK_OK);

  // training side
  n0 = launches;
  EXPECT(stat_topk_huber_forward(x, 16, 9216, 737, 0.01f, (float*)P, nullptr, nullptr) == SPARK_OK);
  EXPECT(stat_topk_huber_backward(x, x, 16, 9216, 737, 0.01f, (float*)P, nullptr) == SPARK_OK);
  EXPECT(launches == n0 + 2);
  EXPECT(stat_topk_huber_forward(x, 16, 9216, 737, 0.f, (float*)P, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk_huber_forward(x, 16, 9216, 737, INFINITY, (float*)P, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk_huber_forward(x, 16, 9216, 9216, 0.1f, (float*)P, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk_huber_backward(x, nullptr, 16, 9216, 737, 0.1f, (float*)P, nullptr) == SPARK_EINVAL);
  EXPECT(stat_topk_huber_backward(x, x, 16, 70000, 737, 0.1f, (float*)P, nullptr) == SPARK_EUNSUPPORTED);
  EXPECT(stat_topk_huber_backward(nullptr, nullptr, 0, 10, 3, 0.1f, nullptr, nullptr) == SPARK_OK);

  // decode
  spark_ffn_shape s{2304, 9216, 1152, 737, SPARK_BF16};
  std::vector<spark_ffn_weights> layers(40, spark_ffn_weights{P, P + 256, P + 512});
  size_t need = 0;
  EXPECT(spark_ffn_decode_workspace_size(&s, 26, 1, &need) == SPARK_OK && need > 0);
  n0 = launches;
  EXPECT(spark_ffn_decode(&s, layers.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, ws, need, nullptr) == SPARK_OK);
  EXPECT(launches == n0 + 1);
  EXPECT(spark_ffn_decode(&s, layers.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, ws, need - 1, nullptr) ==
         SPARK_EWORKSPACE);
  EXPECT(spark_ffn_decode(&s, layers.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, (char*)ws + 8, need, nullptr) ==
         SPARK_EWORKSPACE);
  EXPECT(spark_ffn_decode(&s, layers.data(), 26, x, 1, (float*)P, NAN, nullptr, ws, need, nullptr) == SPARK_EINVAL);
  std::vector<spark_ffn_weights> bad = layers;
  bad[7].v = P + 520;  // not 16-byte aligned
  EXPECT(spark_ffn_decode(&s, bad.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, ws, need, nullptr) == SPARK_EINVAL);
  spark_ffn_shape s2 = s;
  s2.r = 1148;  // r not whole 16-byte chunks of bf16
  EXPECT(spark_ffn_decode_workspace_size(&s2, 26, 1, &need) == SPARK_EINVAL);
  s2 = s;
  s2.wdtype = (spark_dtype)5;
  EXPECT(spark_ffn_decode_workspace_size(&s2, 26, 1, &need) == SPARK_EUNSUPPORTED);
  EXPECT(spark_ffn_decode_tags(26, 1) == 77 && spark_ffn_decode_tags(40, 2) == 2 * (120 - 2));
  EXPECT(spark_ffn_decode_tags(0, 1) == -1);

  // decode without a workspace: the same checks, sizes within the built-in scratch
  n0 = launches;
  EXPECT(spark_ffn_decode_noalloc(&s, layers.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, nullptr) == SPARK_OK);
  EXPECT(launches == n0 + 1);
  EXPECT(spark_ffn_decode_noalloc(&s, bad.data(), 26, x, 1, (float*)P, 1e-6f, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(spark_ffn_decode_noalloc(&s, layers.data(), 0, x, 1, (float*)P, 1e-6f, nullptr, nullptr) == SPARK_EINVAL);
  EXPECT(spark_ffn_decode_noalloc_max_bytes() == spark::kNoAllocScratchBytes);
  // more than one launch of layers needs 8 T d_model bytes more: too many tokens exceed the scratch
  EXPECT(spark_ffn_decode_noalloc(&s, layers.data(), 40, x, 1, (float*)P, 1e-6f, nullptr, nullptr) == SPARK_OK);
  {
    const int64_t T = (int64_t)(spark::kNoAllocScratchBytes / (8 * s.d_model)) + 1;
    EXPECT(spark_ffn_decode_workspace_size(&s, 40, T, &need) == SPARK_OK && need > spark::kNoAllocScratchBytes);
    EXPECT(spark_ffn_decode_noalloc(&s, layers.data(), 40, x, T, (float*)P, 1e-6f, nullptr, nullptr) ==
           SPARK_EUNSUPPORTED);
  }
  EXPECT(spark_ffn_decode_noalloc(&s, layers.data(), 26, x, 0, (float*)P, 1e-6f, nullptr, nullptr) == SPARK_OK);

  // batched decode
  EXPECT(spark_ffn_decode_batched_workspace_size(&s, 8, &need) == SPARK_OK);
  EXPECT(spark_ffn_decode_batched(&s, layers.data(), 26, x, 8, (float*)P, 1e-6f, nullptr, ws, need, nullptr) ==
         SPARK_OK);
  EXPECT(spark_ffn_decode_batched_workspace_size(&s, 9, &need) == SPARK_EUNSUPPORTED);

  // prefill
  EXPECT(spark_ffn_prefill_workspace_size(&s, 4096, &need) == SPARK_OK);
  EXPECT(spark_ffn_prefill(&s, layers.data(), P, 4096, (float*)P, nullptr, ws, need, nullptr) == SPARK_OK);
  EXPECT(spark_ffn_prefill(&s, layers.data(), P + 2, 4096, (float*)P, nullptr, ws, need, nullptr) == SPARK_EINVAL);
  EXPECT(spark_ffn_prefill(&s, layers.data(), P, -1, (float*)P, nullptr, ws, need, nullptr) == SPARK_EINVAL);

  EXPECT(spark_ffn_prefill_gathered_workspace_size(&s, 4096, &need) == SPARK_OK && need > 0);
  EXPECT(spark_ffn_prefill_gathered(&s, layers.data(), P, 4096, (float*)P, nullptr, ws, need, nullptr) == SPARK_OK);
  EXPECT(spark_ffn_prefill_gathered(&s, layers.data(), P, 4096, (float*)(P + 4), nullptr, ws, need, nullptr) ==
         SPARK_EINVAL);
  EXPECT(spark_ffn_prefill_gathered(&s, layers.data(), P, 4096, (float*)P, nullptr, ws, need / 2, nullptr) ==
         SPARK_EWORKSPACE);
  EXPECT(spark_ffn_prefill_scores(&s, layers.data(), P, 4096, (float*)P, nullptr) == SPARK_OK);
  EXPECT(spark_ffn_prefill_scores(&s, layers.data(), P + 4, 4096, (float*)P, nullptr) == SPARK_EINVAL);
  EXPECT(spark_hbm_read_probe(P, 1 << 20, (float*)P, nullptr) == SPARK_OK);
  EXPECT(spark_hbm_read_probe(P, 1000, (float*)P, nullptr) == SPARK_EINVAL);

  // attention decode and prefill
  EXPECT(spark_attn_workspace_size(8, 4, 32768, 256, 128, 256, &need) == SPARK_OK);
  EXPECT(spark_attn_decode(P, P, P, P, 8, 4, 32768, 256, 128, 256, (float*)P, counts, nullptr, 0, nullptr, ws, need,
                           nullptr) == SPARK_OK);
  EXPECT(spark_attn_workspace_size(8, 3, 100, 256, 128, 256, &need) == SPARK_EINVAL);
  size_t need0 = 0, need1 = 0;
  EXPECT(spark_attn_prefill_workspace_size(4096, 8, 4, 256, 128, 256, 0, &need0) == SPARK_OK);
  EXPECT(spark_attn_prefill_workspace_size(4096, 8, 4, 256, 128, 256, 512, &need1) == SPARK_OK && need1 > need0);
  EXPECT(spark_attn_prefill(P, P, P, P, 4096, 8, 4, 256, 128, 256, (float*)P, counts, counts, 512, nullptr, ws,
                            need0, nullptr) == SPARK_EWORKSPACE);
  EXPECT(spark_attn_prefill(P, P, P, P, 4096, 8, 4, 256, 128, 256, (float*)P, counts, counts, 512, nullptr, ws,
                            need1, nullptr) == SPARK_OK);
  EXPECT(spark_attn_prefill(P, P, P, P, 4096, 8, 4, 256, 128, 256, (float*)P, counts, nullptr, 512, nullptr, ws,
                            need0, nullptr) == SPARK_OK);
  EXPECT(spark_attn_prefill(P, P, P, P, 16385, 8, 4, 256, 128, 256, (float*)P, counts, nullptr, 0, nullptr, ws,
                            need1, nullptr) == SPARK_EUNSUPPORTED);

  for (int st = -5; st <= 1; ++st) EXPECT(spark_status_string(st) != nullptr);
  std::printf("api driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
