// Spark FFN decode for a batch of B independent tokens, layer by layer: one
// pass over K1 per layer serves the whole batch, and the K2 and V rows of a
// neuron are read once for all the tokens that select it (the union of the
// per-token selected sets).
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", items
// "Spark FFN" and "Statistical Top-k"): per token and layer
// y = V (GELU(StatTopk(K1^T q[:r])) (.) (K2^T q[r:])), and between layers
// q <- y / sqrt(mean(y^2) + eps); the same computation as spark_ffn_decode,
// with the tokens of the batch processed together instead of one after the
// other.
//
// Per layer three kernels on the stream (a fourth writes the trace when one
// is asked for):
//   bpred: workgroup g owns 32 neurons; it reads their K1 rows once and forms
//          the scores of all B tokens (q[:r] of every token in LDS, each
//          token's RMS scale from its own sum of squares), and the per-token
//          (mean, M2) of its 32 scores;
//   bgate: theta per token from all workgroups' (mean, M2) (two plain sums,
//          fixed order), then per owned neuron the tokens that select it; the
//          K2 row of a neuron selected by any token is read once and dotted
//          with each selecting token's q[r:]; the neurons selected by any
//          token are listed with their B gated values GELU(h - theta) * dot
//          (0 for the tokens that do not select them);
//   bv:    workgroup w owns a range of output columns; it walks every list
//          entry, reads that neuron's V row segment once and accumulates it
//          into the B outputs, then sums over threads in a fixed order.
#include "common.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kBNeur = 32;  // neurons per workgroup of bpred and bgate (eight groups of four)

struct BatchArgs {
  const void* k1t;
  const void* k2t;
  const void* v;
  int d_model, d_ff, r, B;
  float z, eps;
  const float* yin;  // [B][d_model] layer input (prenorm: a layer output to normalise)
  int prenorm;
  float* H;          // [B][d_ff] scores
  float* P;          // [G][B][2] per-workgroup (mean, M2) of the scores
  float* scale;      // [B] RMS scale of the layer input
  float* theta;      // [B]
  int32_t* lcount;   // [G] entries of each workgroup's list
  int32_t* lidx;     // [G][kBNeur] neurons selected by any token
  float* lval;       // [G][kBNeur][B] their gated values
  float* yout;       // [B][d_model] layer output
};

// Sum over the 32 lanes of each half-wave; every lane of the half gets it.
__device__ __forceinline__ float half_sum(float v) {
  v = row16_sum(v);
  return v + __shfl_xor(v, 16, kWave);
}

// ---------------------------------------------------------------- bpred
template <typename W, int BM>
__global__ __launch_bounds__(256) void bpred(const BatchArgs a) {
  constexpr int CN = Chunk<W>::N;
  extern __shared__ float qs[];  // [B][r]: q[:r] of every token (unscaled)
  __shared__ float red[4][BM];
  __shared__ float hs[BM][kBNeur];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model, r = a.r;
  const int n0 = blockIdx.x * kBNeur;
  // token inputs: q[:r] to LDS, sum of squares of the whole row
  for (int b = 0; b < B; ++b) {
    const float* y = a.yin + (size_t)b * d;
    float ss = 0.f;
    for (int c = 4 * tid; c < d; c += 4 * 256) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(y + c);
      if (c < r) *reinterpret_cast<f32x4*>(qs + (size_t)b * r + c) = x;
      ss += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
    }
    ss = wave_sum_dpp(ss);
    if (lane == 0) red[wv][b] = ss;
  }
  __syncthreads();
  float sc[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b)
    sc[b] = (b < B && a.prenorm)
                ? 1.f / sqrtf((((red[0][b] + red[1][b]) + red[2][b]) + red[3][b]) / (float)d + a.eps)
                : 1.f;
  if (blockIdx.x == 0 && tid == 0)
#pragma unroll
    for (int b = 0; b < BM; ++b)
      if (b < B) a.scale[b] = sc[b];
  // scores: group gi (a half-wave) takes neurons n0 + 4 gi + u; lane l of the
  // half takes the 16-byte chunks l, l + 32, ... of their K1 rows
  const int gi = tid >> 5, l32 = tid & 31;
  const int CK = r / CN;
  const size_t rowb = (size_t)r * sizeof(W);
  float acc[4][BM];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[u][b] = 0.f;
  const char* k1 = (const char*)a.k1t;
  int nv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) nv[u] = min(n0 + 4 * gi + u, a.d_ff - 1);  // rows past d_ff: read a valid row, not stored
  for (int c = l32; c < CK; c += 32) {
    float wf[4][CN];
#pragma unroll
    for (int u = 0; u < 4; ++u) Chunk<W>::widen(load16(k1 + (size_t)nv[u] * rowb + (size_t)c * 16), wf[u]);
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      if (b < B) {
        float qv[CN];
#pragma unroll
        for (int e4 = 0; e4 < CN / 4; ++e4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(qs + (size_t)b * r + c * CN + 4 * e4);
          qv[4 * e4] = x.x;
          qv[4 * e4 + 1] = x.y;
          qv[4 * e4 + 2] = x.z;
          qv[4 * e4 + 3] = x.w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < CN; ++e) s += wf[u][e] * qv[e];
          acc[u][b] += s;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      const float t = half_sum(acc[u][b]);
      if (l32 == 0 && b < B) hs[b][4 * gi + u] = t * sc[b];
    }
  __syncthreads();
  // scores out, and each token's (mean, M2) over the owned neurons
  const int nown = min(kBNeur, a.d_ff - n0);
  for (int b = wv; b < B; b += 4) {
    const bool own = lane < nown;
    const float h = own ? hs[b][lane] : 0.f;
    if (own) a.H[(size_t)b * a.d_ff + n0 + lane] = h;
    const float mean = wave_sum_dpp(h) / (float)nown;
    const float dv = own ? h - mean : 0.f;
    const float m2 = wave_sum_dpp(dv * dv);
    if (lane == 0) {
      a.P[((size_t)blockIdx.x * B + b) * 2] = mean;
      a.P[((size_t)blockIdx.x * B + b) * 2 + 1] = m2;
    }
  }
}

// ---------------------------------------------------------------- bgate
template <typename W, int BM>
__global__ __launch_bounds__(256) void bgate(const BatchArgs a) {
  constexpr int CN = Chunk<W>::N;
  extern __shared__ float qs[];  // [B][d - r]: q[r:] of every token, scaled
  __shared__ float th[BM];
  __shared__ float cs[BM][kBNeur];
  __shared__ int sel[kBNeur];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model, r = a.r, rc = d - r;
  const int n0 = blockIdx.x * kBNeur, G = gridDim.x;
  // theta of every token: the mean over all d_ff scores, then their sum of
  // squared deviations, from the per-workgroup (mean, M2) (fixed order)
  for (int b = wv; b < B; b += 4) {
    float s1 = 0.f;
    for (int g = lane; g < G; g += 64) {
      const float n = (float)min(kBNeur, a.d_ff - g * kBNeur);
      s1 += n * a.P[((size_t)g * B + b) * 2];
    }
    const float mu = wave_sum_dpp(s1) / (float)a.d_ff;
    float s2 = 0.f;
    for (int g = lane; g < G; g += 64) {
      const float n = (float)min(kBNeur, a.d_ff - g * kBNeur);
      const float dm = a.P[((size_t)g * B + b) * 2] - mu;
      s2 += a.P[((size_t)g * B + b) * 2 + 1] + n * dm * dm;
    }
    const float m2 = wave_sum_dpp(s2);
    if (lane == 0) th[b] = mu + sqrtf(m2 / (float)a.d_ff) * a.z;
  }
  for (int b = 0; b < B; ++b) {
    const float s = a.scale[b];
    for (int c = 4 * tid; c < rc; c += 4 * 256) {
      f32x4 x = *reinterpret_cast<const f32x4*>(a.yin + (size_t)b * d + r + c);
      x.x *= s;
      x.y *= s;
      x.z *= s;
      x.w *= s;
      *reinterpret_cast<f32x4*>(qs + (size_t)b * rc + c) = x;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < B) a.theta[tid] = th[tid];
  // group gi: neurons n0 + 4 gi + u; the tokens selecting each, then one read
  // of the K2 row of a neuron selected by any of them
  const int gi = tid >> 5, l32 = tid & 31;
  const int CK = rc / CN;
  const size_t rowb = (size_t)rc * sizeof(W);
  const char* k2 = (const char*)a.k2t;
  float hv[4][BM];
  uint32_t sm[4];
  int nv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = n0 + 4 * gi + u;
    nv[u] = min(n, a.d_ff - 1);
    sm[u] = 0;
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      hv[u][b] = (b < B) ? a.H[(size_t)b * a.d_ff + nv[u]] : 0.f;
      sm[u] |= (b < B && n < a.d_ff && hv[u][b] > th[b]) ? 1u << b : 0u;
    }
  }
  float acc[4][BM];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[u][b] = 0.f;
  const uint32_t any = sm[0] | sm[1] | sm[2] | sm[3];
  if (any) {
    for (int c = l32; c < CK; c += 32) {
      float wf[4][CN];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (sm[u]) Chunk<W>::widen(load16(k2 + (size_t)nv[u] * rowb + (size_t)c * 16), wf[u]);
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        if ((any >> b) & 1u) {
          float qv[CN];
#pragma unroll
          for (int e4 = 0; e4 < CN / 4; ++e4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(qs + (size_t)b * rc + c * CN + 4 * e4);
            qv[4 * e4] = x.x;
            qv[4 * e4 + 1] = x.y;
            qv[4 * e4 + 2] = x.z;
            qv[4 * e4 + 3] = x.w;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if ((sm[u] >> b) & 1u) {
              float s = 0.f;
#pragma unroll
              for (int e = 0; e < CN; ++e) s += wf[u][e] * qv[e];
              acc[u][b] += s;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      const float t = half_sum(acc[u][b]);
      if (l32 == 0 && b < B) cs[b][4 * gi + u] = ((sm[u] >> b) & 1u) ? gelu_tanh(hv[u][b] - th[b]) * t : 0.f;
    }
    if (l32 == 0) sel[4 * gi + u] = (int)sm[u];
  }
  __syncthreads();
  // the workgroup's list: the neurons selected by any token, ascending
  if (wv == 0) {
    const bool on = lane < kBNeur && sel[lane < kBNeur ? lane : 0] != 0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(on);
    const int pos = mbcnt64(m);
    if (on) {
      a.lidx[(size_t)blockIdx.x * kBNeur + pos] = n0 + lane;
      for (int b = 0; b < B; ++b) a.lval[((size_t)blockIdx.x * kBNeur + pos) * B + b] = cs[b][lane];
    }
    if (lane == 0) a.lcount[blockIdx.x] = __builtin_popcountll(m);
  }
}

// ---------------------------------------------------------------- bv
// Workgroup w owns the 16-byte column chunks [w NCH, (w + 1) NCH) of the
// output.  Thread t walks the lists of workgroups t, t + 256, ... of bgate
// and accumulates its share of each token's columns; the shares are summed
// over lanes (transposing reduction) and waves in a fixed order.
template <typename W, int BM, int NCH>
__global__ __launch_bounds__(256) void bv(const BatchArgs a, int G2) {
  constexpr int CN = Chunk<W>::N;
  constexpr int NV = BM * NCH * CN;  // accumulators per thread: token-major, then column
  static_assert(NV <= 64 && (NV & (NV - 1)) == 0, "one transposing reduction of at most 64 columns");
  __shared__ float part[4][NV];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model;
  const int nchunks = d / CN;
  const int ch0 = blockIdx.x * NCH;
  const int nch = min(NCH, nchunks - ch0);
  const size_t rowb = (size_t)d * sizeof(W);
  const char* vb = (const char*)a.v + (size_t)ch0 * 16;
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  for (int g = tid; g < G2; g += 256) {
    const int cnt = a.lcount[g];
    for (int e0 = 0; e0 < cnt; e0 += 4) {
      u32x4 raw[4][NCH];
      int n[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) n[k] = e0 + k < cnt ? a.lidx[(size_t)g * kBNeur + e0 + k] : -1;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int hh = 0; hh < NCH; ++hh)
          if (n[k] >= 0 && hh < nch) raw[k][hh] = load16(vb + (size_t)n[k] * rowb + hh * 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (n[k] < 0) continue;
        const float* val = a.lval + ((size_t)g * kBNeur + e0 + k) * B;
#pragma unroll
        for (int hh = 0; hh < NCH; ++hh) {
          if (hh >= nch) continue;
          float wf[CN];
          Chunk<W>::widen(raw[k][hh], wf);
#pragma unroll
          for (int b = 0; b < BM; ++b) {
            if (b < B) {
              const float c = val[b];
#pragma unroll
              for (int i = 0; i < CN; ++i) acc[(b * NCH + hh) * CN + i] += c * wf[i];
            }
          }
        }
      }
    }
  }
  int col;
  const float s = wave_colsum<NV>(acc, lane, col);
  if ((lane & (64 / NV - 1)) == 0) part[wv][col] = s;
  __syncthreads();
  if (tid < NV) {
    const int b = tid / (NCH * CN), rem = tid % (NCH * CN);
    const int hh = rem / CN;
    if (b < B && hh < nch) {
      const float y = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
      a.yout[(size_t)b * d + (size_t)(ch0 + hh) * CN + rem % CN] = y;
    }
  }
}

// ---------------------------------------------------------------- trace
// One workgroup per token: the selected list of the layer (scores above
// theta, ascending), its length, theta and the normalised layer input.
__global__ __launch_bounds__(256) void btrace(const BatchArgs a, int32_t* counts, int32_t* idx, int64_t cap,
                                              float* theta_out, float* q_in, int64_t row0, int64_t row_stride) {
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x, d_ff = a.d_ff;
  const float th = a.theta[b];
  const size_t trow = (size_t)row0 + (size_t)b * row_stride;
  const float* h = a.H + (size_t)b * d_ff;
  // thread t takes the contiguous range [t L, (t + 1) L)
  const int L = (d_ff + 255) / 256;
  const int i0 = min(tid * L, d_ff), i1 = min(i0 + L, d_ff);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += h[i] > th ? 1 : 0;
  const int incl = wave_incl_scan_dpp(c);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += wtot[w];
  int pos = base + incl - c;
  if (idx)
    for (int i = i0; i < i1; ++i)
      if (h[i] > th) {
        if (pos < cap) idx[trow * cap + pos] = i;
        ++pos;
      }
  if (tid == 0) {
    if (counts) counts[trow] = ((wtot[0] + wtot[1]) + wtot[2]) + wtot[3];
    if (theta_out) theta_out[trow] = th;
  }
  if (q_in) {
    const float s = a.scale[b];
    for (int k = tid; k < a.d_model; k += 256) q_in[trow * a.d_model + k] = a.yin[(size_t)b * a.d_model + k] * s;
  }
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct BatchLayout {
  size_t H, P, scale, theta, lcount, lidx, lval, ybuf, total;
};

static BatchLayout batch_layout(int64_t d_model, int64_t d_ff, int64_t B) {
  const int64_t G = (d_ff + kBNeur - 1) / kBNeur;
  BatchLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, 256);
    return o;
  };
  L.H = take((size_t)B * d_ff * 4);
  L.P = take((size_t)G * B * 2 * 4);
  L.scale = take((size_t)B * 4);
  L.theta = take((size_t)B * 4);
  L.lcount = take((size_t)G * 4);
  L.lidx = take((size_t)G * kBNeur * 4);
  L.lval = take((size_t)G * kBNeur * B * 4);
  L.ybuf = take((size_t)B * d_model * 4);
  L.total = off;
  return L;
}

size_t decode_batched_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t B) {
  return batch_layout(d_model, d_ff, B).total;
}


template <typename W, int BM>
static hipError_t launch_batched_t(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                   const float* q, int64_t B, float* y, float eps, double z,
                                   const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  constexpr int CN = Chunk<W>::N;
  constexpr int NCH = (BM * 2 * CN <= 64) ? 2 : 1;  // output chunks per bv workgroup
  const BatchLayout Lo = batch_layout(s.d_model, s.d_ff, B);
  char* base = (char*)ws;
  const int G = (int)((s.d_ff + kBNeur - 1) / kBNeur);
  const int nchunks = (int)(s.d_model / CN);
  const int G3 = (nchunks + NCH - 1) / NCH;
  // (the entry point keeps both at most kBatchMaxLds bytes)
  const size_t lds1 = (size_t)B * s.r * 4, lds2 = (size_t)B * (s.d_model - s.r) * 4;
  hipError_t e = hipSuccess;
  BatchArgs a;
  a.d_model = (int)s.d_model;
  a.d_ff = (int)s.d_ff;
  a.r = (int)s.r;
  a.B = (int)B;
  a.z = (float)z;
  a.eps = eps;
  a.H = (float*)(base + Lo.H);
  a.P = (float*)(base + Lo.P);
  a.scale = (float*)(base + Lo.scale);
  a.theta = (float*)(base + Lo.theta);
  a.lcount = (int32_t*)(base + Lo.lcount);
  a.lidx = (int32_t*)(base + Lo.lidx);
  a.lval = (float*)(base + Lo.lval);
  float* ybuf = (float*)(base + Lo.ybuf);
  for (int l = 0; l < n_layers; ++l) {
    a.k1t = layers[l].k1t;
    a.k2t = layers[l].k2t;
    a.v = layers[l].v;
    a.yin = l == 0 ? q : ybuf;
    a.prenorm = l == 0 ? 0 : 1;
    a.yout = l == n_layers - 1 ? y : ybuf;
    hipLaunchKernelGGL((bpred<W, BM>), dim3(G), dim3(256), lds1, st, a);
    hipLaunchKernelGGL((bgate<W, BM>), dim3(G), dim3(256), lds2, st, a);
    if (trace && (trace->counts || trace->idx || trace->theta || trace->q_in))
      hipLaunchKernelGGL(btrace, dim3((unsigned)B), dim3(256), 0, st, a, trace->counts, trace->idx,
                         trace->idx ? trace->cap : 0, trace->theta, trace->q_in, (int64_t)l, (int64_t)n_layers);
    // bv overwrites ybuf (the input of this layer) only after bpred, bgate and
    // the trace have read it: they precede it on the stream
    hipLaunchKernelGGL((bv<W, BM, NCH>), dim3(G3), dim3(256), 0, st, a, G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename W>
static hipError_t launch_batched_w(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                   const float* q, int64_t B, float* y, float eps, double z,
                                   const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  if (B <= 1) return launch_batched_t<W, 1>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
  if (B <= 2) return launch_batched_t<W, 2>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
  if (B <= 4) return launch_batched_t<W, 4>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
  return launch_batched_t<W, 8>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
}

hipError_t launch_decode_batched(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                 const float* q, int64_t B, float* y, float eps, double z,
                                 const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (s.wdtype == SPARK_BF16) return launch_batched_w<bf16_t>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
  return launch_batched_w<float>(s, layers, n_layers, q, B, y, eps, z, trace, ws, st);
}

}  // namespace spark
