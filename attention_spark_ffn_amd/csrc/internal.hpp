// Launchers behind the C ABI (host side).  Arguments are validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spark_ffn.h"

namespace spark {

// ---------------------------------------------------------------- stat_topk
// theta_in: per-row thresholds to select with (the statistics are then not formed).
hipError_t launch_stat_topk(const float* x, int64_t rows, int64_t d, int64_t ldx, double z, float* vals, int32_t* idx,
                            int64_t cap, int32_t* counts, float* theta, hipStream_t st,
                            const float* theta_in = nullptr);

// ---------------------------------------------------------------- training side (Huber-smoothed stat top-k)
// backward = false: out = y (theta may be null); backward = true: out = dx from dy.
hipError_t launch_stat_topk_huber(bool backward, const float* x, const float* dy, int64_t rows, int64_t d, double z,
                                  float delta, float* out, float* theta, hipStream_t st);

// ---------------------------------------------------------------- decode
// Layers handled by one launch of the persistent decode kernel.
constexpr int kDecodeMaxLayersPerLaunch = 32;
constexpr int kDecodeThreads = 512;
constexpr int kDecodeMaxDModel = 8192;
constexpr int kDecodeMaxNeuronsPerWG = 64;  // one 64-bit selection mask per workgroup
constexpr int kDecodeMaxColsPerWG = 32;

size_t decode_workspace_bytes(int64_t d_model, int64_t d_ff, int n_layers, int64_t T, int grid);
int decode_grid(int64_t d_ff);  // workgroups of the persistent grid on the current device
hipError_t launch_decode(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers, const float* q,
                         int64_t T, float* y, float eps, double z, const spark_ffn_trace* trace, void* ws,
                         hipStream_t st);
// spark_ffn_decode_noalloc: the same kernel on a static per-device scratch of
// kNoAllocScratchBytes (cleared on the first call on a device and before the
// exchange tags would wrap; `tags` is the call's tag count).
constexpr size_t kNoAllocScratchBytes = size_t(2) << 20;
constexpr int kMaxDevices = 64;
hipError_t launch_decode_noalloc(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                 const float* q, int64_t T, float* y, float eps, double z,
                                 const spark_ffn_trace* trace, uint64_t tags, hipStream_t st);

// ---------------------------------------------------------------- batched decode
constexpr int kBatchMax = 8;          // tokens per batch
constexpr int kBatchMaxLds = 65536;   // bytes of q held in LDS per kernel (slots x max(r, d_model - r) x 4)
size_t decode_batched_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t B);
// ws: the buffers after the workspace header; hdr: the header (exchange tags,
// failure record), used by the fused predictor-and-gate kernel.
hipError_t launch_decode_batched(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                 const float* q, int64_t B, float* y, float eps, double z,
                                 const spark_ffn_trace* trace, void* ws, uint64_t* hdr, hipStream_t st);

// ---------------------------------------------------------------- prefill
size_t prefill_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T);
hipError_t launch_prefill(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T, float* Y,
                          double z, const spark_ffn_trace* trace, void* ws, hipStream_t st);
size_t prefill_gathered_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T);
hipError_t launch_prefill_gathered(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T,
                                   float* Y, double z, const spark_ffn_trace* trace, void* ws, hipStream_t st);
hipError_t launch_prefill_scores(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T,
                                 float* H, hipStream_t st);
hipError_t launch_hbm_read_probe(const void* p, size_t bytes, float* sink, hipStream_t st);

// ---------------------------------------------------------------- attention
size_t attn_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn);
size_t attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, bool lists);
hipError_t launch_attn_prefill(const void* q, const void* k1, const void* k2, const void* v, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out, int32_t* counts,
                               int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st);
hipError_t launch_attn_decode(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq, int64_t Hkv,
                              int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double z, float* out,
                              int32_t* counts, int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st);

// device properties (cached per device)
int device_cu_count();

}  // namespace spark
