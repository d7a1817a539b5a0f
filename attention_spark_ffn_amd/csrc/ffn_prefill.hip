// Spark FFN prefill: one layer applied to T tokens at once.
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", items
// "Spark FFN" and "Statistical Top-k"): per token, predictor scores
// h = K1^T q[:r], statistical top-k of h, then
// y = sum over the selected i of GELU(h_i - theta) (K2[:, i] . q[r:]) V[i, :].
//
// gfx950 mapping (every product on the matrix cores, v_mfma_f32_32x32x16_bf16,
// fp32 accumulation):
//   1. H = Q[:, :r] K1 (fp32 scores: rounding them to bf16 would move them by
//      far more than the tie band of the threshold);
//   2. the statistical top-k kernel over the rows of H gives every token's
//      theta (and, when a trace is asked for, its list);
//   3. G = Q[:, r:] K2 with the gate in the epilogue: the tile writes
//      C = GELU(H - theta) * G where H > theta and exact zeros elsewhere, as
//      bf16;
//   4. Y = C V over all neurons.  A neuron that is not selected contributes
//      an exact zero, so this is the same sum as over the selected list; at a
//      selection rate near 8% the dense products on the matrix cores take a
//      fraction of the time of gathering ~737 K2 and V rows per token.  V is
//      first transposed into the workspace so that both operands of every
//      product are read along K.
#include "common.hpp"
#include "gemm.hpp"
#include "internal.hpp"

namespace spark {

// Positions of the caller's list trace past a token's count read -1.
__global__ void pad_lists(const int32_t* __restrict__ counts, int32_t* __restrict__ dst, int64_t cap, int64_t T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * cap) return;
  const int64_t t = i / cap, e = i - t * cap;
  if (e >= counts[t]) dst[i] = -1;
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PrefillLayout {
  size_t H, C, Vt, P, counts, theta, total;
};

constexpr int kOutSplit = 4;  // K splits of the C V product (4096 x 2304: 192 tiles of 256 x 192, 768 with the splits)

static PrefillLayout prefill_layout(int64_t d_model, int64_t d_ff, int64_t T) {
  PrefillLayout L;
  size_t off = 0;
  L.H = off;  // fp32 predictor scores [T][d_ff]
  off += round_up((size_t)T * d_ff * 4, 256);
  L.C = off;  // bf16 gated values [T][d_ff] (zero where not selected)
  off += round_up((size_t)T * d_ff * 2, 256);
  L.Vt = off;  // bf16 V^T [d_model][d_ff]
  off += round_up((size_t)d_model * d_ff * 2, 256);
  L.P = off;  // fp32 partial products of the K splits of C V
  off += round_up((size_t)kOutSplit * T * d_model * 4, 256);
  L.counts = off;
  off += round_up((size_t)T * 4, 256);
  L.theta = off;
  off += round_up((size_t)T * 4, 256);
  L.total = off;
  return L;
}

size_t prefill_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T) {
  return prefill_layout(d_model, d_ff, T).total;
}

hipError_t launch_prefill_scores(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T,
                                 float* H, hipStream_t st) {
  const int M = (int)T, F = (int)s.d_ff, r = (int)s.r, dm = (int)s.d_model;
  return launch_gemm<kEpiStore>(gemm_args((const bf16_t*)Q, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r), 1, 1, st);
}

// Streaming read of `bytes` bytes (a multiple of 16, 16-byte aligned): every
// thread sums the 16-byte chunks it reads, four loads in flight; the sum is
// stored only if it equals a value no finite data gives, so the loads stay
// and nothing is written.
__global__ __launch_bounds__(256) void hbm_read_probe(const u32x4* __restrict__ p, size_t n, float* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  float acc = 0.f;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += __uint_as_float(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc += __uint_as_float(v.x ^ v.y ^ v.z ^ v.w);
  }
  if (__float_as_uint(acc) == 0x7fbadbadu) sink[0] = acc;
}

hipError_t launch_hbm_read_probe(const void* p, size_t bytes, float* sink, hipStream_t st) {
  int cus = device_cu_count();
  if (cus < 1) cus = 256;
  hipLaunchKernelGGL(hbm_read_probe, dim3((unsigned)(8 * cus)), dim3(256), 0, st, (const u32x4*)p, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_prefill(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T, float* Y,
                          double z, const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  const PrefillLayout L = prefill_layout(s.d_model, s.d_ff, T);
  char* base = (char*)ws;
  float* H = (float*)(base + L.H);
  bf16_t* C = (bf16_t*)(base + L.C);
  bf16_t* Vt = (bf16_t*)(base + L.Vt);
  int32_t* counts = (int32_t*)(base + L.counts);
  float* theta = (float*)(base + L.theta);
  const int M = (int)T, F = (int)s.d_ff, r = (int)s.r, dm = (int)s.d_model;
  const bf16_t* Qb = (const bf16_t*)Q;
  // 1. predictor scores
  hipError_t e = launch_gemm<kEpiStore>(gemm_args(Qb, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r), 1, 1, st);
  if (e != hipSuccess) return e;
  // 2. theta per token (and the lists, straight into the trace when asked for)
  const bool want_idx = trace && trace->idx && trace->cap > 0;
  e = launch_stat_topk(H, T, s.d_ff, s.d_ff, z, nullptr, want_idx ? trace->idx : nullptr, want_idx ? trace->cap : 0,
                       counts, theta, st);
  if (e != hipSuccess) return e;
  // 3. gated values C = GELU(H - theta) * (Q[:, r:] K2) on the selected entries
  {
    GemmArgs ga = gemm_args(Qb + r, dm, (const bf16_t*)w.k2t, dm - r, C, F, M, F, dm - r);
    ga.H = H;
    ga.ldh = F;
    ga.r0 = theta;
    e = launch_gemm<kEpiGate>(ga, 1, 1, st);
  }
  if (e != hipSuccess) return e;
  // 4. Y = C V
  // (d_ff is a multiple of 256 and d_model of 8: whole 16-byte chunks both ways)
  hipLaunchKernelGGL(transpose_bf16_x8, dim3((unsigned)((F + 63) / 64), (unsigned)((dm + 63) / 64)), dim3(256), 0, st,
                     (const bf16_t*)w.v, F, dm, Vt, F);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* P = (float*)(base + L.P);
  e = launch_gemm<kEpiStore>(gemm_args(C, F, Vt, F, P, dm, M, dm, F), kOutSplit, 1, st);
  if (e != hipSuccess) return e;
  {
    const int64_t plane = (int64_t)M * dm;  // a multiple of 4 (d_model % 8 == 0)
    hipLaunchKernelGGL(sum_partials, dim3((unsigned)((plane / 4 + 255) / 256)), dim3(256), 0, st, P, kOutSplit, plane,
                       Y);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (trace) {
    if (trace->counts) e = hipMemcpyAsync(trace->counts, counts, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && trace->theta)
      e = hipMemcpyAsync(trace->theta, theta, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && want_idx) {
      const int64_t n = T * trace->cap;
      hipLaunchKernelGGL(pad_lists, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, counts, trace->idx,
                         trace->cap, T);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace spark
