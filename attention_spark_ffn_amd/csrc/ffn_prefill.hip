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

constexpr int GBK = 64;       // K per LDS stage
constexpr int GLD = GBK + 8;  // LDS row length in bf16 (16-byte pad against bank conflicts)

enum { kEpiStore = 0, kEpiGate = 1 };

// D = A[M][K] (bf16, row stride lda) * B^T where B is stored [N][K] (bf16,
// row stride ldb), with K a multiple of 8 and 16-byte aligned rows, over the
// K range of split blockIdx.y (ksplit columns each, a multiple of 64).  Rows of
// A and B past M and N are clamped on load and not stored; K past the end
// reads as zeros.
//
// Workgroup tile (WM*MI*32) x (WN*NI*32): WM x WN waves, each holding MI x NI
// accumulators of v_mfma_f32_32x32x16_bf16 (a 32*MI x 32*NI block).  A wave
// reads MI + NI fragments from LDS per 16 of K for MI*NI MFMAs, so larger
// per-wave blocks cut the LDS traffic per MFMA (64x64 per wave would need the
// whole LDS bandwidth at two workgroups per CU).  K in steps of 64 through
// double-buffered LDS, staged through registers.
//   kEpiStore: C[m][n] (fp32, row stride ldc) = D; with a K split, split s
//              writes its partial to C + s * M * ldc.
//   kEpiGate:  Cg[m][n] (bf16, row stride ldc) = GELU(H - theta[m]) * D where
//              H = H[m][n] (fp32, row stride ldh) > theta[m], else 0.
template <int EPI, int WM, int WN, int MI, int NI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_nt(const bf16_t* __restrict__ A, int lda,
                                                             const bf16_t* __restrict__ B, int ldb,
                                                             void* __restrict__ Cv, int ldc, int M, int N, int K,
                                                             int ksplit, const float* __restrict__ H, int ldh,
                                                             const float* __restrict__ theta) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * MI * 32, BN = WN * NI * 32;
  constexpr int CA = BM * GBK / 8 / NT, CB = BN * GBK / 8 / NT;  // 16-byte chunks per thread per stage
  static_assert(CA * NT * 8 == BM * GBK && CB * NT * 8 == BN * GBK, "tile must split evenly over threads");
  __shared__ alignas(16) bf16_t As[2][BM * GLD];
  __shared__ alignas(16) bf16_t Bs[2][BN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int MT = (M + BM - 1) / BM;
  const int tm = blockIdx.x % MT, tn = blockIdx.x / MT;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = wv / WN, wn = wv % WN;
  const int kbeg = blockIdx.y * ksplit, kend = min(K, kbeg + ksplit);

  // Chunks past K are loaded from column 0 and replaced by zeros only when
  // stored to LDS, after the MFMAs of the current stage, so the loads stay in
  // flight across those MFMAs.
  u32x4 ra[CA], rb[CB];
  int kload = 0;
  auto gload = [&](int k0) {
    kload = k0;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const int k = k0 + kc * 8;
      ra[i] = load16(A + (size_t)min(m0 + row, M - 1) * lda + (k < kend ? k : 0));
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const int k = k0 + kc * 8;
      rb[i] = load16(B + (size_t)min(n0 + row, N - 1) * ldb + (k < kend ? k : 0));
    }
  };
  auto sstore = [&](int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(&As[buf][row * GLD + kc * 8]) = kload + kc * 8 < kend ? ra[i] : zero;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(&Bs[buf][row * GLD + kc * 8]) = kload + kc * 8 < kend ? rb[i] : zero;
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (kend - kbeg + GBK - 1) / GBK;
  gload(kbeg);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kbeg + (kt + 1) * GBK);
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 16) {
      const int ko = kk + (lane >> 5) * 8;  // lanes 0-31: k 0..7, lanes 32-63: k 8..15
      bf16x8 a[MI], b[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * MI * 32 + i * 32 + (lane & 31)) * GLD + ko]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * NI * 32 + j * 32 + (lane & 31)) * GLD + ko]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
  float* Cf = reinterpret_cast<float*>(Cv) + (size_t)blockIdx.y * M * ldc;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    float th[16];
    if (EPI == kEpiGate) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        th[r] = theta[min(m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), M - 1)];
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * NI * 32 + j * 32 + (lane & 31);
      float hv[16];
      if (EPI == kEpiGate) {  // all 16 score loads of the block before any use
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          hv[r] = H[(size_t)min(m, M - 1) * ldh + min(n, N - 1)];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) {
          if (EPI == kEpiStore) {
            Cf[(size_t)m * ldc + n] = acc[i][j][r];
          } else {
            const float c = hv[r] > th[r] ? gelu_tanh(hv[r] - th[r]) * acc[i][j][r] : 0.f;
            reinterpret_cast<bf16_t*>(Cv)[(size_t)m * ldc + n] = f32_to_bf16(c);
          }
        }
      }
    }
  }
}

// Y[m][n] = sum over s < S of P[s][m][n] (fixed order), fp32 [M][N] planes.
__global__ void sum_partials(const float* __restrict__ P, int S, int64_t plane, float* __restrict__ Y) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= plane) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(P + i);
  for (int s = 1; s < S; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(P + (int64_t)s * plane + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<f32x4*>(Y + i) = acc;
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
  size_t H, C, Vt, P, counts, theta, total;
};

constexpr int kOutSplit = 2;  // K splits of the C V product (its tile grid alone is ~2.25 tiles per CU)

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

// Tile configuration of the prefill products: 128 x 128 per workgroup, four
// waves of 64 x 64.  (Two waves of 128 x 64, at one wave per SIMD, measured
// slower: too little to hide the LDS and global latencies.)
constexpr int kWM = 2, kWN = 2, kMI = 2, kNI = 2;
constexpr int kBM = kWM * kMI * 32, kBN = kWN * kNI * 32;

template <int EPI>
static hipError_t launch_gemm(const bf16_t* A, int lda, const bf16_t* B, int ldb, void* C, int ldc, int M, int N,
                              int K, int splits, const float* H, int ldh, const float* theta, hipStream_t st) {
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  int ksplit = (K + splits - 1) / splits;
  ksplit = (ksplit + GBK - 1) / GBK * GBK;
  hipLaunchKernelGGL((gemm_bf16_nt<EPI, kWM, kWN, kMI, kNI>), dim3(tiles, splits), dim3(kWM * kWN * 64), 0, st, A,
                     lda, B, ldb, C, ldc, M, N, K, ksplit, H, ldh, theta);
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
  hipError_t e = launch_gemm<kEpiStore>(Qb, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r, 1, nullptr, 0, nullptr, st);
  if (e != hipSuccess) return e;
  // 2. theta per token (and the lists, straight into the trace when asked for)
  const bool want_idx = trace && trace->idx && trace->cap > 0;
  e = launch_stat_topk(H, T, s.d_ff, s.d_ff, z, nullptr, want_idx ? trace->idx : nullptr, want_idx ? trace->cap : 0,
                       counts, theta, st);
  if (e != hipSuccess) return e;
  // 3. gated values C = GELU(H - theta) * (Q[:, r:] K2) on the selected entries
  e = launch_gemm<kEpiGate>(Qb + r, dm, (const bf16_t*)w.k2t, dm - r, C, F, M, F, dm - r, 1, H, F, theta, st);
  if (e != hipSuccess) return e;
  // 4. Y = C V
  hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)(((F + 63) / 64) * ((dm + 63) / 64))), dim3(256), 0, st,
                     (const bf16_t*)w.v, F, dm, Vt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* P = (float*)(base + L.P);
  e = launch_gemm<kEpiStore>(C, F, Vt, F, P, dm, M, dm, F, kOutSplit, nullptr, 0, nullptr, st);
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
