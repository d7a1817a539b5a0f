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
#include "internal.hpp"

namespace spark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GLD = GBK + 8;  // LDS row length in bf16 (16-byte pad against bank conflicts)

enum { kEpiStore = 0, kEpiGate = 1 };

// D = A[M][K] (bf16, row stride lda) * B^T where B is stored [N][K] (bf16,
// row stride ldb), with K a multiple of 8 and 16-byte aligned rows.  Rows of
// A and B past M and N are clamped on load and not stored; K past the end
// reads as zeros.  128x128 output tile per workgroup (4 waves, 64x64 each),
// K in steps of 64 through double-buffered LDS.
//   kEpiStore: C[m][n] (fp32, row stride ldc) = D.
//   kEpiGate:  Cg[m][n] (bf16, row stride ldc) = GELU(H - theta[m]) * D where
//              H = H[m][n] (fp32, row stride ldh) > theta[m], else 0.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_nt(const bf16_t* __restrict__ A, int lda,
                                                    const bf16_t* __restrict__ B, int ldb, void* __restrict__ Cv,
                                                    int ldc, int M, int N, int K, const float* __restrict__ H,
                                                    int ldh, const float* __restrict__ theta) {
  __shared__ alignas(16) bf16_t As[2][GBM * GLD];
  __shared__ alignas(16) bf16_t Bs[2][GBN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int MT = (M + GBM - 1) / GBM;
  const int tm = blockIdx.x % MT, tn = blockIdx.x / MT;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int wm = wv >> 1, wn = wv & 1;  // 2 x 2 waves, 64 x 64 outputs each

  // global -> register staging: 4 chunks of 16 bytes of A and of B per
  // thread.  Chunks past K are loaded from column 0 and replaced by zeros only
  // when stored to LDS, after the MFMAs of the current step, so the loads stay
  // in flight across those MFMAs.
  u32x4 ra[4], rb[4];
  int kload = 0;
  auto gload = [&](int k0) {
    kload = k0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      const int am = min(m0 + row, M - 1), bn = min(n0 + row, N - 1);
      const int k = k0 + kc * 8;
      const int kk = k < K ? k : 0;
      ra[i] = load16(A + (size_t)am * lda + kk);
      rb[i] = load16(B + (size_t)bn * ldb + kk);
    }
  };
  auto sstore = [&](int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      const bool kin = kload + kc * 8 < K;
      *reinterpret_cast<u32x4*>(&As[buf][row * GLD + kc * 8]) = kin ? ra[i] : zero;
      *reinterpret_cast<u32x4*>(&Bs[buf][row * GLD + kc * 8]) = kin ? rb[i] : zero;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (K + GBK - 1) / GBK;
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
  for (int i = 0; i < 2; ++i) {
    float th[16];
    if (EPI == kEpiGate) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        th[r] = theta[min(m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), M - 1)];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      float hv[16];
      if (EPI == kEpiGate) {  // all 16 score loads of the block before any use
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          hv[r] = H[(size_t)min(m, M - 1) * ldh + min(n, N - 1)];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) {
          if (EPI == kEpiStore) {
            reinterpret_cast<float*>(Cv)[(size_t)m * ldc + n] = acc[i][j][r];
          } else {
            const float c = hv[r] > th[r] ? gelu_tanh(hv[r] - th[r]) * acc[i][j][r] : 0.f;
            reinterpret_cast<bf16_t*>(Cv)[(size_t)m * ldc + n] = f32_to_bf16(c);
          }
        }
      }
    }
  }
}

// Vt[n][k] = V[k][n] for a bf16 [K][N] matrix, 64x64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_bf16(const bf16_t* __restrict__ V, int K, int N,
                                                      bf16_t* __restrict__ Vt) {
  __shared__ bf16_t tile[64][66];
  const int tiles_n = (N + 63) / 64;
  const int tk = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int k0 = tk * 64, n0 = tn * 64, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + 256 * i, r = e >> 6, c = e & 63;
    if (k0 + r < K && n0 + c < N) tile[r][c] = V[(size_t)(k0 + r) * N + n0 + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + 256 * i, r = e >> 6, c = e & 63;  // r: n within tile, c: k within tile
    if (n0 + r < N && k0 + c < K) Vt[(size_t)(n0 + r) * K + k0 + c] = tile[c][r];
  }
}

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
  size_t H, C, Vt, counts, theta, total;
};

static PrefillLayout prefill_layout(int64_t d_model, int64_t d_ff, int64_t T) {
  PrefillLayout L;
  size_t off = 0;
  L.H = off;  // fp32 predictor scores [T][d_ff]
  off += round_up((size_t)T * d_ff * 4, 256);
  L.C = off;  // bf16 gated values [T][d_ff] (zero where not selected)
  off += round_up((size_t)T * d_ff * 2, 256);
  L.Vt = off;  // bf16 V^T [d_model][d_ff]
  off += round_up((size_t)d_model * d_ff * 2, 256);
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

template <int EPI>
static hipError_t launch_gemm(const bf16_t* A, int lda, const bf16_t* B, int ldb, void* C, int ldc, int M, int N,
                              int K, const float* H, int ldh, const float* theta, hipStream_t st) {
  const int tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  hipLaunchKernelGGL(gemm_bf16_nt<EPI>, dim3(tiles), dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K, H, ldh,
                     theta);
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
  hipError_t e = launch_gemm<kEpiStore>(Qb, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r, nullptr, 0, nullptr, st);
  if (e != hipSuccess) return e;
  // 2. theta per token (and the lists, straight into the trace when asked for)
  const bool want_idx = trace && trace->idx && trace->cap > 0;
  e = launch_stat_topk(H, T, s.d_ff, s.d_ff, z, nullptr, want_idx ? trace->idx : nullptr, want_idx ? trace->cap : 0,
                       counts, theta, st);
  if (e != hipSuccess) return e;
  // 3. gated values C = GELU(H - theta) * (Q[:, r:] K2) on the selected entries
  e = launch_gemm<kEpiGate>(Qb + r, dm, (const bf16_t*)w.k2t, dm - r, C, F, M, F, dm - r, H, F, theta, st);
  if (e != hipSuccess) return e;
  // 4. Y = C V
  hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)(((F + 63) / 64) * ((dm + 63) / 64))), dim3(256), 0, st,
                     (const bf16_t*)w.v, F, dm, Vt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gemm<kEpiStore>(C, F, Vt, F, Y, dm, M, dm, F, nullptr, 0, nullptr, st);
  if (e != hipSuccess) return e;
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
