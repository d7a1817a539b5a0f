#include "common.hpp"
#include "internal.hpp"
namespace spark {
size_t prefill_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T) { return 256; }
hipError_t launch_prefill(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T, float* Y,
                          double z, const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  return hipErrorNotSupported;
}
}  // namespace spark
