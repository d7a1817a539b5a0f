#include "common.hpp"
#include "internal.hpp"
namespace spark {
size_t attn_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn) { return 256; }
hipError_t launch_attn_decode(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq, int64_t Hkv,
                              int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double z, float* out,
                              int32_t* counts, int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st) {
  return hipErrorNotSupported;
}
}  // namespace spark
