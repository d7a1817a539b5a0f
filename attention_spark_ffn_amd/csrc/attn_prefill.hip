// Spark attention over a whole prompt (causal prefill).
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", item
// "Spark Attention"): per query head h (KV head g = h / (Hq/Hkv)) the query of
// position t attends over positions j <= t: predictor scores
// s_j = q_t[:r] . k1[g][j], the statistical top-k of s_0..s_t with k_attn
// (every position while t + 1 <= k_attn), softmax of s over the selected set
// and softplus of q_t[r:] . k2[g][j] as the gate on v[g][j].
//
// gfx950 mapping: three dense bf16 products on the matrix cores, causal at
// tile granularity, with the selection applied in an epilogue:
//   1. S = Q[:, h, :r] K1[g]^T (fp32 scores), tiles above the diagonal skipped;
//   2. attn_prefill_rows, one workgroup per (h, t), the row in registers:
//      theta over the t + 1 scores (two exact passes, z = Q(1 - k_attn/(t+1)) from a table
//      computed on the device in fp64), then the largest selected score and
//      the sum of e^(s - max) over the selected;
//   3. W = Q[:, h, r:] K2[g]^T with the epilogue
//      W = e^(s - max)/sum * softplus(.) on the selected j <= t, exact zeros
//      elsewhere (bf16);
//   4. O = W V[g] (V transposed once per call), K stopped at the diagonal.
// An unselected position contributes an exact zero, so the products are the
// same sums as over the selected sets.
#include <cmath>

#include "common.hpp"
#include "gemm.hpp"
#include "internal.hpp"

namespace spark {

// z[n] = Q(1 - k/n) for n in (k, T] (0 elsewhere): bisection on the upper
// tail erfc(z/sqrt 2)/2 = k/n, then Newton steps, in fp64.
__global__ void z_table(int k, int T, float* __restrict__ z) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n > T) return;
  if (n <= k) {
    z[n] = 0.f;
    return;
  }
  const double t = (double)k / (double)n;
  const bool upper = 2 * k <= n;
  const double tt = upper ? t : 1.0 - t;  // solve P(Z > w) = tt for w >= 0
  double lo = 0.0, hi = 1.0;
  while (0.5 * erfc(hi * 0.7071067811865476) > tt && hi < 64.0) hi *= 2.0;
  for (int i = 0; i < 200 && hi - lo > 1e-15 * (1.0 + hi); ++i) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * erfc(mid * 0.7071067811865476) > tt) lo = mid; else hi = mid;
  }
  double w = 0.5 * (lo + hi);
  for (int i = 0; i < 3; ++i) {
    const double pdf = 0.3989422804014327 * exp(-0.5 * w * w);
    if (!(pdf > 0.0)) break;
    w += (0.5 * erfc(w * 0.7071067811865476) - tt) / pdf;
  }
  z[n] = (float)(upper ? w : -w);
}

// Fixed-order sum / max over the 256 threads.
__device__ __forceinline__ float rows_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_sum_dpp(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  const float t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}
__device__ __forceinline__ float rows_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

// One workgroup per (h, t): row t of head h's scores, positions 0..t, held
// in registers (thread i takes the 16-byte chunks i, i + 256, ...; PER values
// per thread cover rows up to 1024 PER), read from memory once.
template <int PER>
__global__ __launch_bounds__(256) void attn_prefill_rows(const float* __restrict__ S, int T, int ldt, int Hq,
                                                         int k_attn,
                                                         const float* __restrict__ ztab, float* __restrict__ rth,
                                                         float* __restrict__ rmx, float* __restrict__ rl,
                                                         int32_t* __restrict__ counts, float* __restrict__ theta) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int h = blockIdx.x / T, t = blockIdx.x % T, n = t + 1;
  const float* s = S + ((size_t)h * T + t) * ldt;
  const bool dense = n <= k_attn;
  // chunks start below n <= ldt (a multiple of 8), so a whole chunk is inside the row
  float v[PER];
  bool ok[PER];
#pragma unroll
  for (int c = 0; c < PER / 4; ++c) {
    const int j = 4 * (tid + 256 * c);
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (j < n) x = *reinterpret_cast<const f32x4*>(s + j);
    v[4 * c] = x.x;
    v[4 * c + 1] = x.y;
    v[4 * c + 2] = x.z;
    v[4 * c + 3] = x.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) ok[4 * c + e] = j + e < n;
  }
  float th = -INFINITY;
  if (!dense) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) a += ok[i] ? v[i] : 0.f;
    const float mean = rows_sum(a, red) / (float)n;
    float b = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float d = v[i] - mean;
      b += ok[i] ? d * d : 0.f;
    }
    const float m2 = rows_sum(b, red);
    th = mean + sqrtf(m2 / (float)n) * ztab[n];
  }
  float mx = -INFINITY;
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool on = ok[i] && v[i] > th;
    mx = on ? fmaxf(mx, v[i]) : mx;
    c += on ? 1 : 0;
  }
  mx = rows_max(mx, red);
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) l += (ok[i] && v[i] > th) ? __expf(v[i] - mx) : 0.f;
  l = rows_sum(l, red);
  const int cnt = (int)rows_sum((float)c, red);  // exact: counts stay far below 2^24
  if (tid == 0) {
    const size_t i = (size_t)h * T + t;
    rth[i] = th;
    rmx[i] = mx;
    rl[i] = l;
    if (counts) counts[(size_t)t * Hq + h] = cnt;
    if (theta) theta[(size_t)t * Hq + h] = dense ? NAN : th;
  }
}

// Columns [c0, ld) of `rows` bf16 rows (ld apart) set to zero: the padding of
// W and V^T past T, which the K loop of O = W V reads in 16-byte chunks.
__global__ void zero_pad_bf16(bf16_t* __restrict__ p, int64_t rows, int ld, int c0) {
  const int w = ld - c0;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * w) return;
  p[(i / w) * ld + c0 + i % w] = 0;
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct AttnPrefillLayout {
  size_t S, W, Vt, rth, rmx, rl, z, total;
};

static AttnPrefillLayout attn_prefill_layout(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd) {
  const int64_t LT = (T + 7) & ~(int64_t)7;
  AttnPrefillLayout L;
  size_t off = 0;
  L.S = off;  // fp32 scores [Hq][T][LT]
  off += round_up((size_t)Hq * T * LT * 4, 256);
  L.W = off;  // bf16 gated weights [Hq][T][LT]
  off += round_up((size_t)Hq * T * LT * 2, 256);
  L.Vt = off;  // bf16 V^T [Hkv][hd][LT]
  off += round_up((size_t)Hkv * hd * LT * 2, 256);
  L.rth = off;
  off += round_up((size_t)Hq * T * 4, 256);
  L.rmx = off;
  off += round_up((size_t)Hq * T * 4, 256);
  L.rl = off;
  off += round_up((size_t)Hq * T * 4, 256);
  L.z = off;
  off += round_up((size_t)(T + 1) * 4, 256);
  L.total = off;
  return L;
}

size_t attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd) {
  return attn_prefill_layout(T, Hq, Hkv, hd).total;
}

hipError_t launch_attn_prefill(const void* q, const void* k1, const void* k2, const void* v, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out, int32_t* counts,
                               float* theta, void* ws, hipStream_t st) {
  const AttnPrefillLayout L = attn_prefill_layout(T, Hq, Hkv, hd);
  char* base = (char*)ws;
  float* S = (float*)(base + L.S);
  bf16_t* W = (bf16_t*)(base + L.W);
  bf16_t* Vt = (bf16_t*)(base + L.Vt);
  float* rth = (float*)(base + L.rth);
  float* rmx = (float*)(base + L.rmx);
  float* rl = (float*)(base + L.rl);
  float* ztab = (float*)(base + L.z);
  const int Ti = (int)T, H = (int)Hq, G = (int)(Hq / Hkv), D = (int)hd, R = (int)r, RC = (int)(hd - r);
  const int LT = (Ti + 7) & ~7;  // row stride of S, W and V^T: 16-byte aligned rows
  const bf16_t* Q = (const bf16_t*)q;
  hipLaunchKernelGGL(z_table, dim3((unsigned)((T + 1 + 255) / 256)), dim3(256), 0, st, (int)k_attn, Ti, ztab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 1. scores
  {
    GemmArgs a = gemm_args(Q, H * D, (const bf16_t*)k1, R, S, LT, Ti, Ti, R);
    a.sA = D;
    a.sB = (int64_t)T * R;
    a.bgroup = G;
    a.sC = (int64_t)T * LT;
    a.causal = kCausalTiles;
    e = launch_gemm<kEpiStore>(a, 1, H, st);
    if (e != hipSuccess) return e;
  }
  // 2. per-row threshold, largest selected score, softmax denominator
  {
    const dim3 g((unsigned)(H * T)), b(256);
    if (Ti <= 1024)
      hipLaunchKernelGGL(attn_prefill_rows<4>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta);
    else if (Ti <= 2048)
      hipLaunchKernelGGL(attn_prefill_rows<8>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta);
    else if (Ti <= 4096)
      hipLaunchKernelGGL(attn_prefill_rows<16>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta);
    else if (Ti <= 8192)
      hipLaunchKernelGGL(attn_prefill_rows<32>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta);
    else
      hipLaunchKernelGGL(attn_prefill_rows<64>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. gated weights
  {
    GemmArgs a = gemm_args(Q + r, H * D, (const bf16_t*)k2, RC, W, LT, Ti, Ti, RC);
    a.sA = D;
    a.sB = (int64_t)T * RC;
    a.bgroup = G;
    a.sC = (int64_t)T * LT;
    a.H = S;
    a.ldh = LT;
    a.sH = (int64_t)T * LT;
    a.r0 = rth;
    a.r1 = rmx;
    a.r2 = rl;
    a.sR = T;
    a.causal = kCausalTiles;
    e = launch_gemm<kEpiAttn>(a, 1, H, st);
    if (e != hipSuccess) return e;
  }
  // 4. O = W V
  for (int64_t gi = 0; gi < Hkv; ++gi) {
    hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)(((T + 63) / 64) * ((hd + 63) / 64))), dim3(256), 0, st,
                       (const bf16_t*)v + (size_t)gi * T * hd, Ti, D, Vt + (size_t)gi * hd * LT, LT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (LT != Ti) {
    const int64_t nw = (int64_t)H * T * (LT - Ti), nv = (int64_t)Hkv * hd * (LT - Ti);
    hipLaunchKernelGGL(zero_pad_bf16, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st, W, (int64_t)H * T, LT,
                       Ti);
    hipLaunchKernelGGL(zero_pad_bf16, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, st, Vt, (int64_t)Hkv * hd,
                       LT, Ti);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    GemmArgs a = gemm_args(W, LT, Vt, LT, out, H * D, Ti, D, Ti);
    a.sA = (int64_t)T * LT;
    a.sB = (int64_t)hd * LT;
    a.bgroup = G;
    a.sC = D;
    a.causal = kCausalK;
    e = launch_gemm<kEpiStore>(a, 1, H, st);
  }
  return e;
}

}  // namespace spark
