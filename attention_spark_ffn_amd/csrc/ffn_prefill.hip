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
//      far more than the tie band of the threshold); the epilogue also writes
//      each row's mean and sum of squared deviations over every wave's column
//      tile, so the statistics need no second pass over the 4 T d_ff bytes
//      of H;
//   2. theta per token from those tile moments (Chan et al.'s combination,
//      in a fixed order); when a trace is asked for, the selection pass lists
//      each token's neurons with that same theta;
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

// theta of each row from the shifted sums of its column tiles (wcols columns
// each, the last one possibly shorter; tile p holds {s, S1, S2} with
// S1 = sum (x - s), S2 = sum (x - s)^2): mean_p = s + S1 / n_p and
// M2_p = S2 - S1^2 / n_p, then mean = sum_p n_p mean_p / N and
// M2 = sum_p (M2_p + n_p (mean_p - mean)^2) (Chan et al.'s combination);
// one wave per row, fixed order.
__global__ __launch_bounds__(256) void theta_from_parts(const f32x4* __restrict__ parts, int T, int nparts, int wcols,
                                                        int N, float z, float* __restrict__ theta) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const f32x4* pr = parts + (size_t)row * nparts;
  auto part = [&](int p, float& n, float& mean, float& m2) {
    const f32x4 q = pr[p];
    n = (float)min(wcols, N - p * wcols);
    mean = q.x + q.y / n;
    m2 = fmaxf(q.z - q.y * q.y / n, 0.f);
  };
  float s1 = 0.f;
  for (int p = lane; p < nparts; p += 64) {
    float n, mp, m2p;
    part(p, n, mp, m2p);
    s1 += n * mp;
  }
  const float mean = wave_sum_dpp(s1) / (float)N;
  float s2 = 0.f;
  for (int p = lane; p < nparts; p += 64) {
    float n, mp, m2p;
    part(p, n, mp, m2p);
    const float dv = mp - mean;
    s2 += m2p + n * dv * dv;
  }
  const float m2 = wave_sum_dpp(s2);
  if (lane == 0) theta[row] = mean + sqrtf(m2 / (float)N) * z;
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
  size_t H, C, Vt, P, counts, theta, parts, total;
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
  L.parts = off;  // per-row moments of the score columns' wave tiles (at most d_ff / 64 + 1 per row)
  off += round_up((size_t)T * (d_ff / 64 + 1) * 16, 256);
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
  // 1. predictor scores and the moments of their column tiles
  f32x4* parts = (f32x4*)(base + L.parts);
  GemmArgs sa = gemm_args(Qb, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r);
  sa.stats = parts;
  const int wcols = gemm_wave_cols<kEpiStats>(sa, 1, 1);
  hipError_t e = launch_gemm<kEpiStats>(sa, 1, 1, st);
  if (e != hipSuccess) return e;
  // 2. theta per token; with a trace, the counts and lists selected with it
  hipLaunchKernelGGL(theta_from_parts, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, (const f32x4*)parts, M,
                     (F + wcols - 1) / wcols, wcols, F, (float)z, theta);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool want_idx = trace && trace->idx && trace->cap > 0;
  if (trace && (trace->counts || want_idx)) {
    e = launch_stat_topk(H, T, s.d_ff, s.d_ff, z, nullptr, want_idx ? trace->idx : nullptr,
                         want_idx ? trace->cap : 0, counts, nullptr, st, theta);
    if (e != hipSuccess) return e;
  }
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
      hipLaunchKernelGGL(pad_lists, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const int32_t*)counts,
                         trace->idx, trace->cap, T);
      e = hipGetLastError();
    }
  }
  return e;
}

// ---------------------------------------------------------------- gathered variant
// The K2 and V steps as the method states them: per token only the selected
// neurons' K2 rows (k2t, neuron-contiguous) and V rows are read.  One
// workgroup per token (256 threads): q_t widened into LDS; rows of 16 lanes
// form the K2 dots of the listed neurons (each lane 16-byte chunks of the
// row, all loads of a row issued before any is used) and the gated values
// c_e = GELU(m_e) * g_e replace m_e in the token's list; then thread j
// accumulates the 16-byte
// column chunks j, j + 256, ... of y over the list in ascending order (eight
// V rows in flight), a fixed order, so results are deterministic.
constexpr int kGatherMaxDModel = 8192;

__global__ __launch_bounds__(256) void prefill_gather(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ k2t,
                                                      const bf16_t* __restrict__ v, const int32_t* __restrict__ idx,
                                                      float* __restrict__ mval, const int32_t* __restrict__ counts,
                                                      int dm, int r, int cap, float* __restrict__ Y) {
  __shared__ float qs[kGatherMaxDModel];  // q_t widened
  const int t = blockIdx.x, tid = threadIdx.x;
  const bf16_t* qt = Q + (size_t)t * dm;
  for (int c = tid; c < dm; c += 256) qs[c] = bf16_to_f32(qt[c]);
  const int n = counts[t];
  const int32_t* it = idx + (size_t)t * cap;
  float* mt = mval + (size_t)t * cap;  // m_e in, c_e out
  float* cs = mt;
  __syncthreads();
  // K2 dots: row of 16 lanes per neuron, 16 neurons per pass
  const int K2C = (dm - r) / 8, l16 = tid & 15, grp = tid >> 4;
  const float* qr = qs + r;
  for (int e0 = 0; e0 < n; e0 += 16) {
    const int e = e0 + grp;
    const int i = it[min(e, n - 1)];
    const char* row = (const char*)(k2t + (size_t)i * (dm - r));
    float acc = 0.f;
    for (int c0 = 0; c0 < K2C; c0 += 16 * 9) {
      u32x4 raw[9];
#pragma unroll
      for (int u = 0; u < 9; ++u) raw[u] = load16(row + (size_t)min(c0 + l16 + 16 * u, K2C - 1) * 16);
#pragma unroll
      for (int u = 0; u < 9; ++u) {
        const int cc = c0 + l16 + 16 * u;
        float wf[8];
        Chunk<bf16_t>::widen(raw[u], wf);
        const float* qq = qr + (cc < K2C ? cc : 0) * 8;
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a += wf[j] * qq[j];
        acc += cc < K2C ? a : 0.f;
      }
    }
    acc = row16_sum(acc);
    if (l16 == 0 && e < n) cs[e] = gelu_tanh(mt[e]) * acc;
  }
  __syncthreads();
  // V: y[cols] = sum over the list (ascending) of c_e V[i_e][cols]
  const int VC = dm / 8;
  for (int ch = tid; ch < VC; ch += 256) {
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int e = 0;
    for (; e + 8 <= n; e += 8) {
      u32x4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = load16(v + (size_t)it[e + u] * dm + (size_t)ch * 8);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float wf[8];
        Chunk<bf16_t>::widen(raw[u], wf);
        const float c = cs[e + u];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] += c * wf[j];
      }
    }
    for (; e < n; ++e) {
      float wf[8];
      Chunk<bf16_t>::widen(load16(v + (size_t)it[e] * dm + (size_t)ch * 8), wf);
      const float c = cs[e];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] += c * wf[j];
    }
    float* yo = Y + (size_t)t * dm + (size_t)ch * 8;
    *reinterpret_cast<f32x4*>(yo) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(yo + 4) = f32x4{y[4], y[5], y[6], y[7]};
  }
}

struct GatherLayout {
  size_t H, parts, theta, counts, idx, m, total;
};

static GatherLayout gather_layout(int64_t d_ff, int64_t T) {
  GatherLayout L;
  size_t off = 0;
  L.H = off;  // fp32 predictor scores [T][d_ff]
  off += round_up((size_t)T * d_ff * 4, 256);
  L.parts = off;
  off += round_up((size_t)T * (d_ff / 64 + 1) * 16, 256);
  L.theta = off;
  off += round_up((size_t)T * 4, 256);
  L.counts = off;
  off += round_up((size_t)T * 4, 256);
  L.idx = off;  // selected neurons of each token, ascending [T][d_ff]
  off += round_up((size_t)T * d_ff * 4, 256);
  L.m = off;  // their soft-threshold values h - theta [T][d_ff]
  off += round_up((size_t)T * d_ff * 4, 256);
  L.total = off;
  return L;
}

size_t prefill_gathered_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t T) {
  (void)d_model;
  return gather_layout(d_ff, T).total;
}

hipError_t launch_prefill_gathered(const spark_ffn_shape& s, const spark_ffn_weights& w, const void* Q, int64_t T,
                                   float* Y, double z, const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  const GatherLayout L = gather_layout(s.d_ff, T);
  char* base = (char*)ws;
  float* H = (float*)(base + L.H);
  f32x4* parts = (f32x4*)(base + L.parts);
  float* theta = (float*)(base + L.theta);
  int32_t* counts = (int32_t*)(base + L.counts);
  int32_t* idx = (int32_t*)(base + L.idx);
  float* m = (float*)(base + L.m);
  const int M = (int)T, F = (int)s.d_ff, r = (int)s.r, dm = (int)s.d_model;
  // 1. predictor scores and their column-tile moments, theta per token
  GemmArgs sa = gemm_args((const bf16_t*)Q, dm, (const bf16_t*)w.k1t, r, H, F, M, F, r);
  sa.stats = parts;
  const int wcols = gemm_wave_cols<kEpiStats>(sa, 1, 1);
  hipError_t e = launch_gemm<kEpiStats>(sa, 1, 1, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(theta_from_parts, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, (const f32x4*)parts, M,
                     (F + wcols - 1) / wcols, wcols, F, (float)z, theta);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. each token's list (ascending) and soft-threshold values, selected with that theta
  e = launch_stat_topk(H, T, F, F, z, m, idx, F, counts, nullptr, st, theta);
  if (e != hipSuccess) return e;
  // 3. the selected neurons' K2 dots and V rows, per token
  hipLaunchKernelGGL(prefill_gather, dim3((unsigned)T), dim3(256), 0, st, (const bf16_t*)Q, (const bf16_t*)w.k2t,
                     (const bf16_t*)w.v, (const int32_t*)idx, m, (const int32_t*)counts, dm, r, F, Y);
  e = hipGetLastError();
  if (e != hipSuccess || !trace) return e;
  if (trace->counts) e = hipMemcpyAsync(trace->counts, counts, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && trace->theta) e = hipMemcpyAsync(trace->theta, theta, (size_t)T * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && trace->idx && trace->cap > 0) {
    e = hipMemcpy2DAsync(trace->idx, (size_t)trace->cap * 4, idx, (size_t)F * 4,
                         (size_t)(trace->cap < F ? trace->cap : F) * 4, (size_t)T, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) {
      const int64_t n = T * trace->cap;
      hipLaunchKernelGGL(pad_lists, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const int32_t*)counts,
                         trace->idx, trace->cap, T);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace spark
