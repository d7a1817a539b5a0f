// Spark FFN prefill: one layer applied to T tokens at once.
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", items
// "Spark FFN" and "Statistical Top-k"): per token, predictor scores
// h = K1^T q[:r], statistical top-k of h, then only the selected neurons' K2
// columns and V rows: y = sum_i GELU(h_i - theta) (K2[:, i] . q[r:]) V[i, :].
//
// gfx950 mapping:
//   1. predictor_gemm: H = Q[:, :r] K1 for all tokens as a dense bf16 GEMM on
//      the matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation and fp32
//      scores (rounding the scores to bf16 would move them by far more than the
//      tie band of the threshold).  128x128 output tile per workgroup, K in
//      steps of 64 through double-buffered LDS.
//   2. the statistical top-k kernel over the rows of H (one workgroup per
//      token), giving each token's ascending neuron list and x - theta values;
//   3. prefill_gather: one workgroup per token forms the gated values
//      c_i = GELU(m_i) (K2^T q[r:])_i of its selected neurons, then y from
//      their V rows (fixed summation order).
#include "common.hpp"
#include "internal.hpp"

namespace spark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GLD = GBK + 8;  // LDS row length in bf16 (16-byte pad against bank conflicts)

// C[M][N] (fp32, row stride ldc) = A[M][K] (bf16, row stride lda) * B^T where
// B is stored [N][K] (bf16, row stride ldb).  Requires N % 128 == 0,
// K % 64 == 0, 16-byte aligned rows; rows of A past M are clamped on load and
// not stored.
__global__ __launch_bounds__(256) void predictor_gemm(const bf16_t* __restrict__ A, int lda,
                                                      const bf16_t* __restrict__ B, int ldb, float* __restrict__ C,
                                                      int ldc, int M, int N, int K) {
  __shared__ alignas(16) bf16_t As[2][GBM * GLD];
  __shared__ alignas(16) bf16_t Bs[2][GBN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int MT = (M + GBM - 1) / GBM;
  const int tm = blockIdx.x % MT, tn = blockIdx.x / MT;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int wm = wv >> 1, wn = wv & 1;  // 2 x 2 waves, 64 x 64 outputs each

  // global -> register staging: 4 chunks of 16 bytes of A and of B per thread
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      const int am = min(m0 + row, M - 1);
      ra[i] = load16(A + (size_t)am * lda + k0 + kc * 8);
      rb[i] = load16(B + (size_t)(n0 + row) * ldb + k0 + kc * 8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(&As[buf][row * GLD + kc * 8]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][row * GLD + kc * 8]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / GBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * GBK);
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 16) {
      const int ko = kk + (lane >> 5) * 8;  // lanes 0-31: k 0..7, lanes 32-63: k 8..15
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 64 + i * 32 + (lane & 31)) * GLD + ko]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * 64 + j * 32 + (lane & 31)) * GLD + ko]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < M) C[(size_t)m * ldc + n] = acc[i][j][r];
      }
}

constexpr int kGatherSeg = 4096;  // selected entries per LDS segment

// One workgroup per token: gated values of the selected neurons, then y.
__global__ __launch_bounds__(256) void prefill_gather(const bf16_t* __restrict__ Q, int d_model, int r,
                                                      const bf16_t* __restrict__ k2t, const bf16_t* __restrict__ v,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ vals,
                                                      const int32_t* __restrict__ counts, int cap,
                                                      float* __restrict__ Y) {
  __shared__ alignas(16) float qr[kDecodeMaxDModel];
  __shared__ float cs[kGatherSeg];
  __shared__ int is[kGatherSeg];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rc = d_model - r, K2C = rc / 8, VC = d_model / 8;
  const int n = min(counts[t], cap);
  for (int j = tid; j < rc; j += 256) qr[j] = bf16_to_f32(Q[(size_t)t * d_model + r + j]);
  __syncthreads();
  for (int s0 = 0; s0 < n || s0 == 0; s0 += kGatherSeg) {
    const int ns = min(kGatherSeg, n - s0);
    for (int e = tid; e < ns; e += 256) is[e] = idx[(size_t)t * cap + s0 + e];
    __syncthreads();
    // K2 gather-dot: wave wv takes entries wv, wv + 4, ...; three rows per pass
    for (int e0 = wv; e0 < ns; e0 += 12) {
      float sacc[3] = {0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < K2C; c0 += 64) {
        u32x4 raw[3];
        const int cc = min(c0 + lane, K2C - 1);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const int e = min(e0 + 4 * u, ns - 1);
          raw[u] = load16(k2t + (size_t)is[e] * rc + (size_t)cc * 8);
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          float wf[8];
          Chunk<bf16_t>::widen(raw[u], wf);
          const f32x4* qq = reinterpret_cast<const f32x4*>(qr + cc * 8);
          const f32x4 q0 = qq[0], q1 = qq[1];
          const float a = wf[0] * q0.x + wf[1] * q0.y + wf[2] * q0.z + wf[3] * q0.w + wf[4] * q1.x + wf[5] * q1.y +
                          wf[6] * q1.z + wf[7] * q1.w;
          sacc[u] += (c0 + lane < K2C) ? a : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const float g = wave_sum_dpp(sacc[u]);
        const int e = e0 + 4 * u;
        if (lane == 0 && e < ns) cs[e] = gelu_tanh(vals[(size_t)t * cap + s0 + e]) * g;
      }
    }
    __syncthreads();
    // V rows: thread owns 8 consecutive output columns, entries in ascending order
    for (int vc = tid; vc < VC; vc += 256) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = s0 == 0 ? 0.f : Y[(size_t)t * d_model + vc * 8 + i];
      int e = 0;
      for (; e + 8 <= ns; e += 8) {
        u32x4 raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = load16(v + (size_t)is[e + u] * d_model + (size_t)vc * 8);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float wf[8];
          Chunk<bf16_t>::widen(raw[u], wf);
          const float c = cs[e + u];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += c * wf[i];
        }
      }
      for (; e < ns; ++e) {
        float wf[8];
        Chunk<bf16_t>::widen(load16(v + (size_t)is[e] * d_model + (size_t)vc * 8), wf);
        const float c = cs[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += c * wf[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) Y[(size_t)t * d_model + vc * 8 + i] = acc[i];
    }
    __syncthreads();
    if (n == 0) break;
  }
}

// Copy the first `cap` list entries of every token into the caller's trace
// (-1 past the token's count).
__global__ void copy_lists(const int32_t* __restrict__ src, int src_cap, const int32_t* __restrict__ counts,
                           int32_t* __restrict__ dst, int64_t dst_cap, int64_t T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * dst_cap) return;
  const int64_t t = i / dst_cap, e = i - t * dst_cap;
  dst[i] = (e < src_cap && e < counts[t]) ? src[t * src_cap + e] : -1;
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PrefillLayout {
  size_t H, vals, idx, counts, theta, total;
};

static PrefillLayout prefill_layout(int64_t d_ff, int64_t T) {
  PrefillLayout L;
  size_t off = 0;
  L.H = off;
  off += round_up((size_t)T * d_ff * 4, 256);
  L.vals = off;
  off += round_up((size_t)T * d_ff * 4, 256);
  L.idx = off;
  off += round_up((size_t)T * d_ff * 4, 256);
  L.counts = off;
  off += round_up((size_t)T * 4, 256);
  L.theta = off;
  off += round_up((size_t)T * 4, 256);
  L.total = off;
  return L;
}

size_t prefill_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T) {
  (void)d_model;
  return prefill_layout(d_ff, T).total;
}

hipError_t launch_prefill(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T, float* Y,
                          double z, const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  const PrefillLayout L = prefill_layout(s.d_ff, T);
  char* base = (char*)ws;
  float* H = (float*)(base + L.H);
  float* vals = (float*)(base + L.vals);
  int32_t* idx = (int32_t*)(base + L.idx);
  int32_t* counts = (int32_t*)(base + L.counts);
  float* theta = (float*)(base + L.theta);
  const int M = (int)T, N = (int)s.d_ff, K = (int)s.r, dm = (int)s.d_model;
  const int tiles = ((M + GBM - 1) / GBM) * (N / GBN);
  hipLaunchKernelGGL(predictor_gemm, dim3(tiles), dim3(256), 0, st, (const bf16_t*)Q, dm, (const bf16_t*)w.k1t, K, H,
                     N, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_stat_topk(H, T, s.d_ff, s.d_ff, z, vals, idx, s.d_ff, counts, theta, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_gather, dim3((unsigned)T), dim3(256), 0, st, (const bf16_t*)Q, dm, K,
                     (const bf16_t*)w.k2t, (const bf16_t*)w.v, idx, vals, counts, N, Y);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (trace) {
    if (trace->counts) e = hipMemcpyAsync(trace->counts, counts, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && trace->theta)
      e = hipMemcpyAsync(trace->theta, theta, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && trace->idx && trace->cap > 0) {
      const int64_t n = T * trace->cap;
      hipLaunchKernelGGL(copy_lists, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx, N, counts,
                         trace->idx, trace->cap, T);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace spark
