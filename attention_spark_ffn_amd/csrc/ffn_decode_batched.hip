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
// Per layer, on the stream (one more kernel writes the trace when one is
// asked for):
//   bpred: workgroup g owns up to 40 neurons; it reads their K1 rows once and
//          forms the scores of all B tokens (q[:r] of every token in LDS, each
//          token's RMS scale from the previous layer's sums of squares), and
//          the per-token (mean, M2) of its scores;
//   bgate: theta per token from all workgroups' (mean, M2) (two plain sums,
//          fixed order), then per owned neuron the tokens that select it; the
//          K2 row of a neuron selected by any token is read once and dotted
//          with each selecting token's q[r:]; it writes the B gated values
//          GELU(h - theta) * dot of its neurons (0 for the tokens that do not
//          select them) and the mask of its neurons selected by any token;
//   bfused: bpred and bgate in one launch whose workgroups exchange the
//          (mean, M2) as tagged words while they run (bf16 weights, both
//          products on the matrix cores, a grid the device holds at once);
//   bv (one token) or bv2 + breduce (more): the union of the selected sets
//          times V, each union neuron's V row segment read once for all the
//          tokens, summed over slices in a fixed order, with each token's sum
//          of squares for the next layer's RMS scale.
#include <type_traits>

#include "common.hpp"
#include "exchange.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kBSlots = 40;    // neurons per workgroup of bpred and bgate at most (ten groups of four)
constexpr int kBThreads = 320;  // threads of bpred and bgate: ten half-waves

// First neuron of workgroup g of G (the G workgroups split d_ff evenly).
__device__ __forceinline__ int nfirst(int g, int d_ff, int G) { return (int)((int64_t)g * d_ff / G); }

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
  uint64_t* umask;   // [G] neurons of each workgroup selected by any token (bit j: its neuron j)
  float* C;          // [d_ff][BM] gated values (0 for a token that does not select the neuron; slots >= B unused)
  float* yout;       // [B][d_model] layer output
  float* ssp;        // [G3][BM] each reduce workgroup's sum of squares of its output columns, per token
  int G3;            // reduce workgroups (column segments)
};

// Sum over the 32 lanes of each half-wave; every lane of the half gets it.
__device__ __forceinline__ float half_sum(float v) {
  v = row16_sum(v);
  return v + __shfl_xor(v, 16, kWave);
}

// Column sums of NV per-lane values (NV a power of two, at most 32) over the
// 32 lanes of each half-wave, all columns at once: at each step a lane hands
// half of its remaining columns to the lane m apart and adds the other half of
// that lane's; after log2(NV) steps each lane holds the partial of one column
// (col = l32 / (32 / NV)) and the remaining steps add over the lanes that
// share it.
template <int NV>
__device__ __forceinline__ float half_colsum(float (&v)[NV], int lane, int& col) {
  constexpr int S = NV >= 32 ? 5 : NV >= 16 ? 4 : NV >= 8 ? 3 : NV >= 4 ? 2 : NV >= 2 ? 1 : 0;
  static_assert((1 << S) == NV, "NV must be a power of two");
  col = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int m = 16 >> s, h = NV >> (s + 1);
    const uint32_t upm = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const uint32_t x = __float_as_uint(v[i]), y = __float_as_uint(v[i + h]);
      const float give = __uint_as_float((x & upm) | (y & ~upm));
      const float keep = __uint_as_float((y & upm) | (x & ~upm));
      v[i] = keep + __shfl_xor(give, m, kWave);
    }
    col += (lane & m) ? h : 0;
  }
  float t = v[0];
#pragma unroll
  for (int m = 16 >> S; m >= 1; m >>= 1) t += __shfl_xor(t, m, kWave);
  return t;
}

// Columns [c0, c0 + n) of every token's input row (n a multiple of 4) into
// LDS at dst[b * n + j], times scale[b] (scale null: unscaled); with ss, the
// per-wave sums of squares of the whole rows (all d columns) into ss[wave][b].
// Every load of a thread is issued before any is used.
template <int BM, int NT>
__device__ __forceinline__ void load_tokens(const float* __restrict__ yin, int B, int d, int c0, int n,
                                            float* __restrict__ dst, const float* scale, float (*ss)[BM]) {
  constexpr int KMAX = 3;  // 16-byte loads per thread and token per round
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lo = ss ? 0 : c0, hi = ss ? d : c0 + n;  // columns read
  for (int base = lo; base < hi; base += 4 * NT * KMAX) {
    f32x4 x[BM][KMAX];
#pragma unroll
    for (int b = 0; b < BM; ++b)
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int c = base + 4 * (tid + NT * k);
        if (b < B && c < hi) x[b][k] = *reinterpret_cast<const f32x4*>(yin + (size_t)b * d + c);
      }
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      if (b >= B) continue;
      const float s = scale ? scale[b] : 1.f;
      float sq = 0.f;
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int c = base + 4 * (tid + NT * k);
        if (c < hi) {
          const f32x4 v = x[b][k];
          if (c >= c0 && c < c0 + n) {
            const f32x4 w = {v.x * s, v.y * s, v.z * s, v.w * s};
            *reinterpret_cast<f32x4*>(dst + (size_t)b * n + (c - c0)) = w;
          }
          sq += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
        }
      }
      if (ss) {
        sq = wave_sum_dpp(sq);
        if (lane == 0) ss[wv][b] += sq;
      }
    }
  }
}

// ---------------------------------------------------------------- products on the matrix cores
// D[n][b] = row_n . q_b for a workgroup's rows (at most 48: three tiles of
// 16) and its token slots (BM <= 8), on v_mfma_f32_16x16x32_bf16 (rows = the
// tile's rows, columns = token slots and parts).  Each fp32 token vector
// enters the bf16 products as three parts, q = hi + mid + lo (hi = bf16(q),
// mid = bf16(q - hi), lo = bf16(q - hi - mid); the two differences are exact,
// and |q - hi - mid - lo| <= 2^-27 |q|): with the bf16 weights exact and the
// products accumulated in fp32 the result keeps the accuracy of fp32
// products.  Two products per K step: columns 0..7 hi and 8..15 mid of the
// token slots, then lo in columns 0..7.  The K range (kq steps of 32) is
// split over the workgroup's NW waves; each wave's partial tiles go to
// part[wave][tile][product][column][row], and mfma_rows_sum adds them in a
// fixed order.
typedef __bf16 bt_bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kMTiles = 3;   // 16-row tiles (kBSlots <= 48)
constexpr int kMSteps = 8;   // K steps of 32 per wave (K <= 32 * kMSteps * waves)
static_assert(kBSlots <= 16 * kMTiles, "a workgroup's rows must fit the tiles");

// The A fragments of this wave: row row[t] (a valid row of the workgroup for
// every lane) of tile t, K steps w * spw + s, elements 8 (lane / 16) .. + 7;
// a tile whose row is not wanted (want[t] false) reads nothing (zeros).
template <int NW>
__device__ __forceinline__ void mfma_rows_load(u32x4 (&fa)[kMTiles][kMSteps], const char* base, size_t rowb,
                                               const int (&row)[kMTiles], const bool (&want)[kMTiles], int kq,
                                               int wv, int lane) {
  const int spw = (kq + NW - 1) / NW;
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) {
    const char* rp = base + (size_t)row[t] * rowb + (size_t)(8 * (lane >> 4)) * sizeof(bf16_t);
#pragma unroll
    for (int s = 0; s < kMSteps; ++s) {
      const int ks = min(wv * spw + min(s, spw - 1), kq - 1);  // steps past the range re-read a valid one (unused)
      fa[t][s] = want[t] ? load16(rp + (size_t)ks * 64) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int BM, int NW>
__device__ __forceinline__ void mfma_rows_products(const u32x4 (&fa)[kMTiles][kMSteps], const float* qs, int K,
                                                   int kq, float (*part)[kMTiles][2][16][16], int wv, int lane) {
  const int spw = (kq + NW - 1) / NW;
  const int n = lane & 15, b = n & 7;
  const bool second = n >= 8, live = b < BM;
  f32x4 acc[kMTiles][2];
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMSteps; ++s) {
    const int ks = wv * spw + s;
    if (s < spw && ks < kq) {
      const float* src = qs + (size_t)(live ? b : 0) * K + 32 * ks + 8 * (lane >> 4);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bt_bf16x8 b0, b1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = live ? v[j] : 0.f;
        const __bf16 hi = (__bf16)x;
        const float r1 = x - (float)hi;
        const __bf16 mid = (__bf16)r1;
        const __bf16 lo = (__bf16)(r1 - (float)mid);
        b0[j] = second ? mid : hi;
        b1[j] = second ? (__bf16)0.f : lo;
      }
#pragma unroll
      for (int t = 0; t < kMTiles; ++t) {
        const bt_bf16x8 af = __builtin_bit_cast(bt_bf16x8, fa[t][s]);
        acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b0, acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b1, acc[t][1], 0, 0, 0);
      }
    }
  }
  // result register i of lane l: row 4 (l / 16) + i, column l % 16
#pragma unroll
  for (int t = 0; t < kMTiles; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<f32x4*>(&part[wv][t][q][lane & 15][4 * (lane >> 4)]) = acc[t][q];
}

// Row j (< 48) of the product for token slot b: the waves' partials of the
// three parts, in a fixed order.
template <int NW>
__device__ __forceinline__ float mfma_rows_sum(float (*part)[kMTiles][2][16][16], int j, int b) {
  const int t = j >> 4, m = j & 15;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += (part[w][t][0][b][m] + part[w][t][0][b + 8][m]) + part[w][t][1][b][m];
  return s;
}

// The matrix-core paths take bf16 weights.
template <typename W>
constexpr bool kMatrixOk = std::is_same<W, bf16_t>::value;

// ---------------------------------------------------------------- bpred
// MF: the scores on the matrix cores (bf16 weights, r a multiple of 32 and at
// most 32 kMSteps waves); otherwise on the vector units.
template <typename W, int BM, bool MF>
__global__ __launch_bounds__(kBThreads) void bpred(const BatchArgs a) {
  constexpr int CN = Chunk<W>::N;
  extern __shared__ float qs[];  // [B][r]: q[:r] of every token (unscaled)
  __shared__ float red[kBThreads / 64][BM];
  __shared__ float hs[BM][kBSlots];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model, r = a.r;
  const int n0 = nfirst(blockIdx.x, a.d_ff, gridDim.x), n1 = nfirst(blockIdx.x + 1, a.d_ff, gridDim.x);
  // scores: group gi (a half-wave) takes neurons n0 + 4 gi + u; lane l of the
  // half takes the 16-byte chunks l, l + 32, ... of their K1 rows, in rounds
  // of kRound chunks per neuron with all loads of a round issued before any
  // is used.  The first round does not depend on the tokens: it is issued
  // before their loads, so the two round trips overlap.
  const int gi = tid >> 5, l32 = tid & 31;
  const int CK = r / CN;
  const size_t rowb = (size_t)r * sizeof(W);
  const char* k1 = (const char*)a.k1t;
  int nv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) nv[u] = min(n0 + 4 * gi + u, n1 - 1);  // slots past the range: a valid row, not stored
  constexpr int kRound = 5;
  constexpr int NW = kBThreads / 64;
  __shared__ float part[NW][kMTiles][2][16][16];  // matrix-core partials
  static_assert(!MF || std::is_same<W, bf16_t>::value, "matrix-core path: bf16 weights");
  constexpr bool mf = MF;
  u32x4 raw[kRound][4];
  u32x4 fa[kMTiles][kMSteps];
  auto issue = [&](int c0) {
#pragma unroll
    for (int k = 0; k < kRound; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = min(c0 + 32 * k, CK - 1);
        raw[k][u] = load16(k1 + (size_t)nv[u] * rowb + (size_t)c * 16);
      }
  };
  if constexpr (mf) {
    int row[kMTiles];
    bool want[kMTiles];
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) {
      row[t] = min(n0 + 16 * t + (lane & 15), n1 - 1);
      want[t] = true;
    }
    mfma_rows_load<NW>(fa, k1, rowb, row, want, r / 32, wv, lane);
  } else {
    issue(l32);
  }
  // each token's RMS scale from the previous layer's per-workgroup sums of
  // squares (half-wave b, fixed order), and q[:r] of every token to LDS
  if (a.prenorm) {
    const int b = tid >> 5, l32 = tid & 31;
    if (b < B) {
      float ss = 0.f;
      for (int w0 = l32; w0 < a.G3; w0 += 32 * 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = w0 + 32 * k < a.G3 ? a.ssp[(size_t)(w0 + 32 * k) * BM + b] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += v[k];
      }
      ss = half_sum(ss);
      if (l32 == 0) red[0][b] = 1.f / sqrtf(ss / (float)d + a.eps);
    }
  }
  for (int i = B * r + tid; i < BM * r; i += kBThreads) qs[i] = 0.f;  // empty token slots
  load_tokens<BM, kBThreads>(a.yin, B, d, 0, r, qs, nullptr, nullptr);
  __syncthreads();
  float sc[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) sc[b] = (b < B && a.prenorm) ? red[0][b] : 1.f;
  if (blockIdx.x == 0 && tid == 0)
#pragma unroll
    for (int b = 0; b < BM; ++b)
      if (b < B) a.scale[b] = sc[b];
  if constexpr (mf) {
    mfma_rows_products<BM, NW>(fa, qs, r, r / 32, part, wv, lane);
    __syncthreads();
    const int nown = n1 - n0;
    for (int i = tid; i < BM * kBSlots; i += kBThreads) {
      const int b = i / kBSlots, j = i % kBSlots;
      if (b < B && j < nown) hs[b][j] = mfma_rows_sum<NW>(part, j, b) * sc[b];
    }
  }
  float acc[4][BM];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[u][b] = 0.f;
  const f32x4* q4 = reinterpret_cast<const f32x4*>(qs);  // r is a multiple of 4
  for (int c0 = l32; !mf && c0 < CK; c0 += 32 * kRound) {
    if (c0 != l32) issue(c0);
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      const int c = c0 + 32 * k;
      if (c >= CK) break;
      float wf[4][CN];
#pragma unroll
      for (int u = 0; u < 4; ++u) Chunk<W>::widen(raw[k][u], wf[u]);
      // every token slot up to BM (slots past B hold zeros: no branches)
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        float qv[CN];
#pragma unroll
        for (int e4 = 0; e4 < CN / 4; ++e4) {
          const f32x4 x = q4[(b * r + c * CN) / 4 + e4];
          qv[4 * e4] = x.x;
          qv[4 * e4 + 1] = x.y;
          qv[4 * e4 + 2] = x.z;
          qv[4 * e4 + 3] = x.w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float sd = 0.f;
#pragma unroll
          for (int e = 0; e < CN; ++e) sd += wf[u][e] * qv[e];
          acc[u][b] += sd;
        }
      }
    }
  }
  if constexpr (!mf) {
    float flat[4 * BM];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int b = 0; b < BM; ++b) flat[u * BM + b] = acc[u][b];
    int col;
    const float t = half_colsum<4 * BM>(flat, lane, col);
    const int u = col / BM, b = col % BM;
    if ((l32 & (32 / (4 * BM) - 1)) == 0 && b < B) hs[b][4 * gi + u] = t * sc[b];
  }
  __syncthreads();
  // scores out, and each token's (mean, M2) over the owned neurons
  const int nown = n1 - n0;  // at most kBSlots
  for (int b = wv; b < B; b += kBThreads / 64) {
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
// MF: the K2 dots on the matrix cores (bf16 weights, d - r a multiple of 32
// and at most 32 kMSteps waves); otherwise on the vector units.
template <typename W, int BM, bool MF>
__global__ __launch_bounds__(kBThreads) void bgate(const BatchArgs a) {
  constexpr int CN = Chunk<W>::N;
  extern __shared__ float qs[];  // [B][d - r]: q[r:] of every token, scaled
  __shared__ float th[BM];
  __shared__ uint32_t sel[kBSlots];
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.B, d = a.d_model, r = a.r, rc = d - r;
  const int G = gridDim.x;
  const int n0 = nfirst(blockIdx.x, a.d_ff, G), n1 = nfirst(blockIdx.x + 1, a.d_ff, G);
  // Everything that does not depend on theta is loaded first, in one round
  // trip: the per-workgroup (mean, M2) of the scores (token b: half-wave b,
  // lanes over workgroups), this group's scores, and q[r:] of every token.
  const int gi = tid >> 5, l32 = tid & 31;
  constexpr int KG = 8;  // workgroups per lane held in registers (one pass when G <= 256)
  const bool one_pass = G <= 32 * KG;
  float mn[KG], m2v[KG];
  if (one_pass && gi < B) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int g = l32 + 32 * k;
      mn[k] = g < G ? a.P[((size_t)g * B + gi) * 2] : 0.f;
      m2v[k] = g < G ? a.P[((size_t)g * B + gi) * 2 + 1] : 0.f;
    }
  }
  float hv[4][BM];
  int nv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    nv[u] = min(n0 + 4 * gi + u, n1 - 1);
#pragma unroll
    for (int b = 0; b < BM; ++b) hv[u][b] = (b < B) ? a.H[(size_t)b * a.d_ff + nv[u]] : 0.f;
  }
  for (int i = B * rc + tid; i < BM * rc; i += kBThreads) qs[i] = 0.f;  // empty token slots
  load_tokens<BM, kBThreads>(a.yin, B, d, r, rc, qs, a.scale, nullptr);
  // theta of every token: the mean over all d_ff scores, then their sum of
  // squared deviations, from the per-workgroup (mean, M2) (fixed order)
  {
    const int b = gi;
    if (b < B) {
      float s1 = 0.f, s2 = 0.f, mu;
      if (one_pass) {
        float nn[KG];
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          const int g = l32 + 32 * k;
          nn[k] = g < G ? (float)(nfirst(g + 1, a.d_ff, G) - nfirst(g, a.d_ff, G)) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < KG; ++k) s1 += nn[k] * mn[k];
        mu = half_sum(s1) / (float)a.d_ff;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          const float dm = mn[k] - mu;
          s2 += nn[k] > 0.f ? m2v[k] + nn[k] * dm * dm : 0.f;
        }
      } else {  // two passes over the partials, KG per lane at a time
        for (int g0 = l32; g0 < G; g0 += 32 * KG) {
          float mn[KG], nn[KG];
#pragma unroll
          for (int k = 0; k < KG; ++k) {
            const int g = g0 + 32 * k;
            mn[k] = g < G ? a.P[((size_t)g * B + b) * 2] : 0.f;
            nn[k] = g < G ? (float)(nfirst(g + 1, a.d_ff, G) - nfirst(g, a.d_ff, G)) : 0.f;
          }
#pragma unroll
          for (int k = 0; k < KG; ++k) s1 += nn[k] * mn[k];
        }
        mu = half_sum(s1) / (float)a.d_ff;
        for (int g0 = l32; g0 < G; g0 += 32 * KG) {
          float mn[KG], m2v[KG], nn[KG];
#pragma unroll
          for (int k = 0; k < KG; ++k) {
            const int g = g0 + 32 * k;
            mn[k] = g < G ? a.P[((size_t)g * B + b) * 2] : 0.f;
            m2v[k] = g < G ? a.P[((size_t)g * B + b) * 2 + 1] : 0.f;
            nn[k] = g < G ? (float)(nfirst(g + 1, a.d_ff, G) - nfirst(g, a.d_ff, G)) : 0.f;
          }
#pragma unroll
          for (int k = 0; k < KG; ++k) {
            const float dm = mn[k] - mu;
            s2 += nn[k] > 0.f ? m2v[k] + nn[k] * dm * dm : 0.f;
          }
        }
      }
      s2 = half_sum(s2);
      if (l32 == 0) th[b] = mu + sqrtf(s2 / (float)a.d_ff) * a.z;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < B) a.theta[tid] = th[tid];
  // group gi: neurons n0 + 4 gi + u; the tokens selecting each, then one read
  // of the K2 row of a neuron selected by any of them
  const int CK = rc / CN;
  const size_t rowb = (size_t)rc * sizeof(W);
  const char* k2 = (const char*)a.k2t;
  uint32_t sm[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    sm[u] = 0;
#pragma unroll
    for (int b = 0; b < BM; ++b)
      sm[u] |= (b < B && n0 + 4 * gi + u < n1 && hv[u][b] > th[b]) ? 1u << b : 0u;
  }
  constexpr int NW = kBThreads / 64;
  // the K2 dots on the matrix cores (the rows of neurons no token selects
  // read as zeros)
  static_assert(!MF || std::is_same<W, bf16_t>::value, "matrix-core path: bf16 weights");
  if constexpr (MF) {
    __shared__ float part[NW][kMTiles][2][16][16];
    const int wv = tid >> 6;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (l32 == 0) sel[4 * gi + u] = sm[u];
    __syncthreads();
    const int nown = n1 - n0;
    int row[kMTiles];
    bool want[kMTiles];
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) {
      const int j = 16 * t + (lane & 15);
      row[t] = min(n0 + j, n1 - 1);
      want[t] = j < nown && j < kBSlots && sel[j < kBSlots ? j : 0] != 0;
    }
    u32x4 fa[kMTiles][kMSteps];
    mfma_rows_load<NW>(fa, k2, rowb, row, want, rc / 32, wv, lane);
    mfma_rows_products<BM, NW>(fa, qs, rc, rc / 32, part, wv, lane);
    __syncthreads();
    // gated values of the owned neurons: C[n][b] (exact 0 for the tokens that
    // do not select n)
    for (int i = tid; i < BM * kBSlots; i += kBThreads) {
      const int b = i / kBSlots, j = i % kBSlots;
      if (b < B && j < nown) {
        const int n = n0 + j;
        const bool on = (sel[j] >> b) & 1u;
        const float g = mfma_rows_sum<NW>(part, j, b);
        a.C[(size_t)n * BM + b] = on ? gelu_tanh(a.H[(size_t)b * a.d_ff + n] - th[b]) * g : 0.f;
      }
    }
    if (tid < 64) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(lane < kBSlots && sel[lane < kBSlots ? lane : 0] != 0);
      if (lane == 0) a.umask[blockIdx.x] = m;
    }
    return;
  }
  float acc[4][BM];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[u][b] = 0.f;
  const uint32_t any = sm[0] | sm[1] | sm[2] | sm[3];
  if (any) {
    const f32x4* q4 = reinterpret_cast<const f32x4*>(qs);  // d - r is a multiple of 4
    constexpr int kRound = 5;
    for (int c0 = l32; c0 < CK; c0 += 32 * kRound) {
      u32x4 raw[kRound][4];
#pragma unroll
      for (int k = 0; k < kRound; ++k)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          raw[k][u] = u32x4{0u, 0u, 0u, 0u};
          if (sm[u]) raw[k][u] = load16(k2 + (size_t)nv[u] * rowb + (size_t)min(c0 + 32 * k, CK - 1) * 16);
        }
#pragma unroll
      for (int k = 0; k < kRound; ++k) {
        const int c = c0 + 32 * k;
        if (c >= CK) break;
        float wf[4][CN];
#pragma unroll
        for (int u = 0; u < 4; ++u) Chunk<W>::widen(raw[k][u], wf[u]);
        // every (neuron, token) pair of the group; unselected pairs are
        // dropped at the end (no branches here; unread K2 rows are zeros)
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          float qv[CN];
#pragma unroll
          for (int e4 = 0; e4 < CN / 4; ++e4) {
            const f32x4 x = q4[(b * rc + c * CN) / 4 + e4];
            qv[4 * e4] = x.x;
            qv[4 * e4 + 1] = x.y;
            qv[4 * e4 + 2] = x.z;
            qv[4 * e4 + 3] = x.w;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float sd = 0.f;
#pragma unroll
            for (int e = 0; e < CN; ++e) sd += wf[u][e] * qv[e];
            acc[u][b] += sd;
          }
        }
      }
    }
  }
  // gated values of the owned neurons: C[n][b] (exact 0 for the tokens that
  // do not select n); the union mask of the workgroup
  {
    float flat[4 * BM];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int b = 0; b < BM; ++b) flat[u * BM + b] = acc[u][b];
    int col;
    const float t = half_colsum<4 * BM>(flat, lane, col);
    const int u = col / BM, b = col % BM, n = n0 + 4 * gi + u;
    // this lane's (neuron, token) pair: its score and selection bit (the
    // registers of pair (u, b) are picked with selects, not indexed)
    float h = 0.f;
    uint32_t smu = 0;
#pragma unroll
    for (int uu = 0; uu < 4; ++uu)
#pragma unroll
      for (int bb = 0; bb < BM; ++bb) {
        h = (uu == u && bb == b) ? hv[uu][bb] : h;
        smu = uu == u ? sm[uu] : smu;
      }
    if ((l32 & (32 / (4 * BM) - 1)) == 0 && b < B && n < n1)
      a.C[(size_t)n * BM + b] = ((smu >> b) & 1u) ? gelu_tanh(h - th[b]) * t : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (l32 == 0) sel[4 * gi + u] = sm[u];
  __syncthreads();
  if (tid < 64) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(lane < kBSlots && sel[lane < kBSlots ? lane : 0] != 0);
    if (lane == 0) a.umask[blockIdx.x] = m;
  }
}

// ---------------------------------------------------------------- bv (one token)
// Workgroup w owns the 16-byte column chunks [w NCH, (w + 1) NCH) of the
// output.  The union of the selected sets (bgate's masks, prefix counts in
// LDS) is split into contiguous runs, one per thread, each walked
// kBvRound neurons at a time with all their loads (the gated values and the
// V row chunks) issued before any is used; the per-thread sums are then added
// over lanes (transposing reduction) and waves in a fixed order.
constexpr int kBvThreads = 512;  // two waves per SIMD: one walks while the other waits on its loads
template <typename W, int BM>
__global__ __launch_bounds__(kBvThreads) void bv(const BatchArgs a, int G2) {
  constexpr int CN = Chunk<W>::N;
  constexpr int kBvRound = BM >= 8 ? 4 : 8;  // union neurons per round of loads
  constexpr int NCH = 2;             // output chunks per workgroup at most
  constexpr int NV1 = BM * CN;       // accumulators per thread and chunk: token-major, then column
  static_assert(NV1 <= 64 && (NV1 & (NV1 - 1)) == 0, "one transposing reduction of at most 64 columns per chunk");
  constexpr int NWV = kBvThreads / 64;
  constexpr int WPT = 2048 / kBvThreads;  // mask words per thread in the prefix count
  __shared__ float part[NWV][NCH][NV1];
  __shared__ float yy[NCH][NV1];
  __shared__ uint64_t um[2048];
  __shared__ int pre[2049];
  __shared__ int wtot[NWV];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model;
  const int nchunks = d / CN;
  // column owner index: the workgroups of one XCD (w = x + 8 j, dealt
  // round-robin) own one contiguous run of chunks, so each cache line of a V
  // row is fetched by one XCD
  const int G3 = gridDim.x;  // at least nchunks / 2: one or two chunks each
  const int o = (G3 % 8 == 0) ? (blockIdx.x & 7) * (G3 / 8) + (blockIdx.x >> 3) : blockIdx.x;
  const int ch0 = (int)((int64_t)o * nchunks / G3);
  const int nch = (int)((int64_t)(o + 1) * nchunks / G3) - ch0;
  const size_t rowb = (size_t)d * sizeof(W);
  const char* vb = (const char*)a.v + (size_t)ch0 * 16;
  // union masks and their exclusive prefix counts (thread t: words WPT t ..)
  int cnt8 = 0;
  uint64_t w8[WPT];
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int g = WPT * tid + k;
    w8[k] = g < G2 ? a.umask[g] : 0ull;
    cnt8 += __builtin_popcountll(w8[k]);
  }
  const int incl = wave_incl_scan_dpp(cnt8);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int run = incl - cnt8;
  for (int w2 = 0; w2 < wv; ++w2) run += wtot[w2];
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int g = WPT * tid + k;
    if (g < 2048) {
      um[g] = w8[k];
      pre[g] = run;
    }
    run += __builtin_popcountll(w8[k]);
  }
  if (tid == kBvThreads - 1) pre[2048] = run;
  __syncthreads();
  const int U = pre[2048];
  float acc[NCH][NV1];
#pragma unroll
  for (int hh = 0; hh < NCH; ++hh)
#pragma unroll
    for (int i = 0; i < NV1; ++i) acc[hh][i] = 0.f;
  // thread t takes the union entries [t U / NT, (t + 1) U / NT): one search
  // for the first, then a walk along the set bits of the masks
  const int e_begin = (int)((int64_t)tid * U / kBvThreads), e_end = (int)((int64_t)(tid + 1) * U / kBvThreads);
  int g = 0;
  uint64_t wbits = 0;
  if (e_begin < e_end) {
    int lo = 0, hi = G2 - 1;  // last workgroup g with pre[g] <= e_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= e_begin) lo = mid; else hi = mid - 1;
    }
    g = lo;
    wbits = um[g];
    for (int k = e_begin - pre[g]; k > 0; --k) wbits &= wbits - 1;  // drop the entries before e_begin
  }
  for (int e0 = e_begin; e0 < e_end; e0 += kBvRound) {
    int n[kBvRound];
#pragma unroll
    for (int k = 0; k < kBvRound; ++k) {
      n[k] = -1;
      if (e0 + k < e_end) {
        while (wbits == 0) wbits = um[++g];
        n[k] = nfirst(g, a.d_ff, G2) + __builtin_ctzll(wbits);
        wbits &= wbits - 1;
      }
    }
    f32x4 cv[kBvRound][(BM + 3) / 4];
    u32x4 raw[kBvRound][NCH];
#pragma unroll
    for (int k = 0; k < kBvRound; ++k) {
      if (n[k] < 0) continue;
      if (BM >= 4) {
#pragma unroll
        for (int j = 0; j < BM / 4; ++j) cv[k][j] = reinterpret_cast<const f32x4*>(a.C + (size_t)n[k] * BM)[j];
      } else {
#pragma unroll
        for (int b = 0; b < BM; ++b) cv[k][0][b] = a.C[(size_t)n[k] * BM + b];
      }
#pragma unroll
      for (int hh = 0; hh < NCH; ++hh)
        if (hh < nch) raw[k][hh] = load16(vb + (size_t)n[k] * rowb + hh * 16);
    }
#pragma unroll
    for (int k = 0; k < kBvRound; ++k) {
      if (n[k] < 0) continue;
#pragma unroll
      for (int hh = 0; hh < NCH; ++hh) {
        if (hh >= nch) continue;
        float wf[CN];
        Chunk<W>::widen(raw[k][hh], wf);
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          const float c = cv[k][b / 4][b % 4];
#pragma unroll
          for (int i = 0; i < CN; ++i) acc[hh][b * CN + i] += c * wf[i];
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < NCH; ++hh) {
    int col;
    const float sum = wave_colsum<NV1>(acc[hh], lane, col);
    if ((lane & (64 / NV1 - 1)) == 0) part[wv][hh][col] = sum;
  }
  __syncthreads();
  if (tid < NCH * NV1) {
    const int hh = tid / NV1, rem = tid % NV1, b = rem / CN;
    float y = 0.f;
    if (b < B && hh < nch) {
      for (int w2 = 0; w2 < NWV; ++w2) y += part[w2][hh][rem];
      a.yout[(size_t)b * d + (size_t)(ch0 + hh) * CN + rem % CN] = y;
    }
    yy[hh][rem] = y * y;
  }
  __syncthreads();
  // each token's sum of squares over the owned columns (fixed order), for the
  // RMS scale of the next layer
  if (tid < BM) {
    float ss = 0.f;
#pragma unroll
    for (int hh = 0; hh < NCH; ++hh)
#pragma unroll
      for (int i = 0; i < CN; ++i) ss += yy[hh][tid * CN + i];
    a.ssp[(size_t)blockIdx.x * BM + tid] = ss;
  }
}

// ---------------------------------------------------------------- bv2 + breduce (two or more tokens)
// The V product by (column block, union slice): workgroup (cb, sp) takes the
// 128-byte line cb of every V row it needs (eight 16-byte chunks) and the
// union neurons of the predictor workgroups [sp G / S, (sp + 1) G / S) (their
// masks only, placed by prefix counts: no search over the whole union).
// Eight lanes read one row's line
// together (lane l: row l / 8 of the wave's eight rows, chunk l % 8), so a
// wave's load instruction covers eight whole lines, and each V row is read by
// one workgroup per line instead of one per 16-byte chunk.  The slice sums go
// to P2[sp][b][column]; breduce adds the slices in a fixed order and forms
// each token's sum of squares for the next layer's RMS scale.
constexpr int kBv2Threads = 256;
constexpr int kBv2Round = 4;      // rows per lane in flight
constexpr int kBv2Rows = 2048;    // union entries whose neurons are resolved into LDS at a time (32 masks)

// Slices per column block: about two workgroups per CU over the whole grid.
static int bv2_slices(int64_t d_model, int cn) {
  const int64_t nblocks = (d_model / cn + 7) / 8;
  int64_t cus = device_cu_count();
  if (cus < 1) cus = 256;
  int64_t S = (2 * cus + nblocks - 1) / nblocks;
  return (int)(S < 1 ? 1 : S > 64 ? 64 : S);
}

// One halving step of octet_colsum: lanes with bit M of the lane index set
// keep the upper K / 2 of their K values, the others the lower, each adding
// the partner's (lane ^ M) matching half.
template <int M, int K, int NV>
__device__ __forceinline__ void octet_step(float (&v)[NV], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int j = 0; j < K / 2; ++j) {
    const float send = up ? v[j] : v[j + K / 2];
    const float recv = __shfl_xor(send, M, kWave);
    v[j] = (up ? v[j + K / 2] : v[j]) + recv;
  }
}
// v[0 .. NV) summed over the eight lanes that share lane % 8, transposing:
// afterwards lane l holds in v[0 .. NV / 8) the sums of the values
// (NV / 8) (l / 8) + j.
template <int NV>
__device__ __forceinline__ void octet_colsum(float (&v)[NV], int lane) {
  static_assert(NV >= 8 && (NV & (NV - 1)) == 0, "a power of two, at least 8");
  octet_step<32, NV, NV>(v, lane);
  octet_step<16, NV / 2, NV>(v, lane);
  octet_step<8, NV / 4, NV>(v, lane);
}

// FOLD (the launches whose predictor-and-gate kernel is bfused): no breduce.
// Each workgroup publishes its slice sums as tagged words at
// X2[block x S + slice][token][column of the block] (the layer's tag, which
// bfused has just stored in the workspace header), and the block's last slice
// -- dispatched after the others, so it only ever waits on workgroups already
// started -- adds the S slices in the same fixed order as breduce, writes y
// and each token's sum of squares over the block's columns to ssp[block].
// Every wait is bounded; on timeout the call is marked failed and the block's
// outputs are NaN.
constexpr int kFoldCols = 64;  // columns of a column block (eight 16-byte bf16 chunks)
template <typename W, int BM, bool FOLD>
__global__ __launch_bounds__(kBv2Threads) void bv2(const BatchArgs a, int G2, int S, float* __restrict__ P2,
                                                   uint64_t* hdr, uint64_t* X2, int layer) {
  constexpr int CN = Chunk<W>::N;
  constexpr int NV = BM * CN < 8 ? 8 : BM * CN;  // accumulators per lane (padded to eight)
  constexpr int NWV = kBv2Threads / 64;
  constexpr int kGrp = kBv2Rows / 64;  // predictor workgroups (64-bit masks) resolved into LDS at a time
  __shared__ uint64_t um[kGrp];
  __shared__ int pre[kGrp];
  __shared__ int s_ns;
  __shared__ int rows[kBv2Rows];
  __shared__ float part[NWV][8][NV];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, d = a.d_model, nchunks = d / CN;
  const int cb = blockIdx.x / S, sp = blockIdx.x % S;
  // this slice: the union neurons of predictor workgroups [g0, g1), in
  // ascending order (each workgroup owns a contiguous neuron range)
  const int g0 = (int)((int64_t)sp * G2 / S), g1 = (int)((int64_t)(sp + 1) * G2 / S);
  // this lane: row rl of each group of eight, chunk c of the block's line
  const int rl = lane >> 3, c = lane & 7, gc = cb * 8 + c;
  const size_t rowb = (size_t)d * sizeof(W);
  const char* vb = (const char*)a.v + (size_t)(gc < nchunks ? gc : nchunks - 1) * 16;
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  for (int gg0 = g0; gg0 < g1; gg0 += kGrp) {
    const int ng = min(kGrp, g1 - gg0);
    __syncthreads();  // the previous group's rows are read
    if (wv == 0) {  // the group's masks and their exclusive prefix counts
      const uint64_t m = lane < ng ? a.umask[gg0 + lane] : 0ull;
      const int cnt = __builtin_popcountll(m);
      const int incl = wave_incl_scan_dpp(cnt);
      if (lane < kGrp) {
        um[lane] = m;
        pre[lane] = incl - cnt;
      }
      if (lane == 63) s_ns = incl;
    }
    __syncthreads();
    // neuron j of workgroup gg0 + w goes to the place of its rank among the
    // group's selected neurons
    for (int p = tid; p < ng * 64; p += kBv2Threads) {
      const int w = p >> 6, j = p & 63;
      const uint64_t m = um[w];
      if ((m >> j) & 1ull)
        rows[pre[w] + __builtin_popcountll(m & ((1ull << j) - 1ull))] = nfirst(gg0 + w, a.d_ff, G2) + j;
    }
    __syncthreads();
    const int ns = s_ns;
    // rows (k NWV + wv) 8 + rl of each pass; a slot past the sub-slice repeats
    // row 0 (in bounds) with weight zero, so a pass has no branches
    for (int p0 = 0; p0 < ns; p0 += kBv2Round * NWV * 8) {
      int n[kBv2Round];
      bool ok[kBv2Round];
#pragma unroll
      for (int k = 0; k < kBv2Round; ++k) {
        const int i = p0 + (k * NWV + wv) * 8 + rl;
        ok[k] = i < ns;
        n[k] = rows[ok[k] ? i : 0];
      }
      f32x4 cv[kBv2Round][(BM + 3) / 4];
      u32x4 raw[kBv2Round];
#pragma unroll
      for (int k = 0; k < kBv2Round; ++k) {
        if (BM >= 4) {
#pragma unroll
          for (int j = 0; j < BM / 4; ++j) cv[k][j] = reinterpret_cast<const f32x4*>(a.C + (size_t)n[k] * BM)[j];
        } else {
#pragma unroll
          for (int b = 0; b < BM; ++b) cv[k][0][b] = a.C[(size_t)n[k] * BM + b];
        }
        raw[k] = load16(vb + (size_t)n[k] * rowb);
      }
#pragma unroll
      for (int k = 0; k < kBv2Round; ++k) {
        float wf[CN];
        Chunk<W>::widen(raw[k], wf);
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          const float cb_ = ok[k] ? cv[k][b / 4][b % 4] : 0.f;
#pragma unroll
          for (int i = 0; i < CN; ++i) acc[b * CN + i] += cb_ * wf[i];
        }
      }
    }
  }
  // sums over the eight rows of a wave, then over the waves (fixed order)
  octet_colsum<NV>(acc, lane);
#pragma unroll
  for (int j = 0; j < NV / 8; ++j) part[wv][c][(lane >> 3) * (NV / 8) + j] = acc[j];
  __syncthreads();
  if constexpr (!FOLD) {
    for (int t = tid; t < 8 * NV; t += kBv2Threads) {
      const int cc = t / NV, idx = t % NV, b = idx / CN, i = idx % CN, gcc = cb * 8 + cc;
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) sum += part[w2][cc][idx];
      if (b < B && gcc < nchunks) P2[((size_t)sp * B + b) * d + (size_t)gcc * CN + i] = sum;
    }
  } else {
    static_assert(!FOLD || 8 * CN == kFoldCols, "the folded reduction takes 16-byte chunks of eight bf16 values");
    __shared__ float own[BM * kFoldCols];
    __shared__ uint32_t s_tag, s_spin;
    __shared__ uint64_t s_fmark;
    if (tid == 0) {
      s_tag = (uint32_t)get_word(hdr);
      s_fmark = (uint64_t)(s_tag - (uint32_t)layer);
      const uint64_t lim = get_word(hdr + 3);  // the host-set test hook bounds every wait
      s_spin = lim ? (uint32_t)lim : (1u << 22);
    }
    __syncthreads();
    const uint32_t tag = s_tag;
    const bool red = sp == S - 1;
    uint64_t* mine = X2 + (size_t)blockIdx.x * (BM * kFoldCols);
    for (int t = tid; t < 8 * NV; t += kBv2Threads) {
      const int cc = t / NV, idx = t % NV, b = idx / CN, i = idx % CN;
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) sum += part[w2][cc][idx];
      if (b < B) {
        if (red)
          own[b * kFoldCols + cc * CN + i] = sum;
        else
          put_tagged(mine + b * kFoldCols + cc * CN + i, sum, tag);
      }
    }
    if (!red) return;
    __syncthreads();
    // output o = token b (o / 64), column o % 64 of the block; a thread takes
    // o = tid + 256 j (j < NO), so each wave's sums of squares belong to one
    // token per j.  The words of up to KP slices of all a thread's outputs
    // are polled in one round.
    constexpr int NO = (BM * kFoldCols + kBv2Threads - 1) / kBv2Threads;
    constexpr int KP = 16;
    const uint64_t* blk = X2 + (size_t)cb * S * (BM * kFoldCols);
    float y[NO];
    bool okall = true;
#pragma unroll
    for (int j = 0; j < NO; ++j) y[j] = 0.f;
    const size_t sstride = (size_t)BM * kFoldCols;  // words between the slices of a block
    static_assert(NO * KP <= 32, "one pending bit per polled word");
    for (int s0 = 0; s0 < S - 1 && okall; s0 += KP) {
      // bit j KP + k: slice s0 + k of output j still without the layer's tag
      uint32_t pend = 0;
#pragma unroll
      for (int j = 0; j < NO; ++j) {
        const int o = tid + kBv2Threads * j;
        if (o < BM * kFoldCols && o / kFoldCols < B)
#pragma unroll
          for (int k = 0; k < KP; ++k)
            if (s0 + k < S - 1) pend |= 1u << (j * KP + k);
      }
      const uint32_t want = pend;
      uint32_t v[NO * KP];
      for (uint32_t spin = 0; pend; ++spin) {
        uint64_t wvv[NO * KP];
#pragma unroll
        for (int i = 0; i < NO * KP; ++i)
          if ((pend >> i) & 1u)
            wvv[i] = get_word(blk + (size_t)(s0 + i % KP) * sstride + tid + kBv2Threads * (i / KP));
#pragma unroll
        for (int i = 0; i < NO * KP; ++i)
          if (((pend >> i) & 1u) && (uint32_t)(wvv[i] >> 32) == tag) {
            v[i] = (uint32_t)wvv[i];
            pend &= ~(1u << i);
          }
        if (!pend) break;
        if (spin > s_spin || ((spin & 1023) == 1023 && get_word(hdr + 1) == s_fmark)) {
          okall = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int i = 0; i < NO * KP; ++i)  // slices in ascending order, as breduce
        if ((want >> i) & 1u) y[i / KP] += __uint_as_float(v[i]);
    }
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int o = tid + kBv2Threads * j;
      const int b = o / kFoldCols, gcol = cb * kFoldCols + o % kFoldCols;
      const bool valid = o < BM * kFoldCols && b < B;
      float yo = valid ? y[j] + own[o] : 0.f;
      if (!okall) yo = __builtin_nanf("");
      if (valid && gcol < d) a.yout[(size_t)b * d + gcol] = yo;
      float ss = valid && gcol < d ? yo * yo : 0.f;
      ss = wave_sum_dpp(ss);
      if (lane == 0 && valid) a.ssp[(size_t)cb * BM + b] = ss;
    }
    if (!okall) raise_failure(hdr, s_fmark);
  }
}

// y[b][:] = sum over the S slices (fixed order), and each token's sum of
// squares over the workgroup's 256 columns (for the next layer's RMS scale).
// One wave per (column segment, token); four slices' loads in flight.
constexpr int kRedCols = 256;
template <int BM>
__global__ __launch_bounds__(64) void breduce(const BatchArgs a, int S, const float* __restrict__ P2) {
  const int b = blockIdx.y, seg = blockIdx.x, lane = threadIdx.x;
  const int B = a.B, d = a.d_model;
  const int c0 = seg * kRedCols + 4 * lane;
  float ss = 0.f;
  if (c0 < d) {  // d is a multiple of 4
    const size_t step = (size_t)B * d;
    const float* p = P2 + (size_t)b * d + c0;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const f32x4*>(p + (size_t)(s + k) * step);
#pragma unroll
      for (int k = 0; k < 4; ++k) y += v[k];
    }
    for (; s < S; ++s) y += *reinterpret_cast<const f32x4*>(p + (size_t)s * step);
    *reinterpret_cast<f32x4*>(a.yout + (size_t)b * d + c0) = y;
    ss = ((y.x * y.x + y.y * y.y) + y.z * y.z) + y.w * y.w;
  }
  ss = wave_sum_dpp(ss);
  if (lane == 0) a.ssp[(size_t)seg * BM + b] = ss;
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

// ---------------------------------------------------------------- bfused
// bpred and bgate as one kernel: a grid the device holds at once (one
// workgroup per CU, checked on the host), the per-workgroup (mean, M2) of the
// scores exchanged as tagged words (device-scope relaxed atomics, replicated
// once per XCD; a reader accepts a word only with this launch's tag, taken
// from the workspace header) instead of across a kernel boundary.  Both
// products on the matrix cores (bf16 weights; r and d - r multiples of 32, at
// most 32 kMSteps waves).  Every wait is bounded: on timeout the launch marks
// the call failed in the header (as the single-token kernel does), writes NaN
// gated values for its neurons and ends; workgroup 0 advances the header's
// tag on every way out.
constexpr int kXRow = 256;  // exchange words are word-major: word k of workgroup g at k * kXRow + g
// bfused loads q[:r] and q[r:] as one 16-byte piece per thread and token
static_assert(4 * kBThreads >= 32 * kMSteps * (kBThreads / 64), "r and d - r up to the products' K must fit");
constexpr int kXRep = 8;    // replicas (one per XCD)

// A failed call's layer: NaN gated values for the owned neurons, all marked
// used (so the V product spreads NaN over every output), and the tag advanced.
template <int BM>
__device__ __forceinline__ void bfused_failed(const BatchArgs& a, uint64_t* hdr, int n0, int nown, uint32_t tag) {
  for (int i = threadIdx.x; i < BM * kBSlots; i += kBThreads) {
    const int b = i / kBSlots, j = i % kBSlots;
    if (b < a.B && j < nown) a.C[(size_t)(n0 + j) * BM + b] = __builtin_nanf("");
  }
  if (threadIdx.x == 0) {
    a.umask[blockIdx.x] = nown >= 64 ? ~0ull : (1ull << nown) - 1;
    if (blockIdx.x == 0) __hip_atomic_store(hdr, (uint64_t)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int BM>
__global__ __launch_bounds__(kBThreads) void bfused(const BatchArgs a, uint64_t* hdr, uint64_t* xs, int xs_stride,
                                                      int layer) {
  constexpr int NW = kBThreads / 64;
  extern __shared__ float dyn[];  // q[:r] of every token slot (unscaled), then q[r:] (scaled)
  __shared__ float red[BM];       // each token's RMS scale
  __shared__ float hs[BM][kBSlots];
  __shared__ float part[NW][kMTiles][2][16][16];
  __shared__ float th[BM];
  __shared__ uint32_t sel[kBSlots];
  __shared__ uint32_t s_tag, s_spin, s_poison;
  __shared__ uint64_t s_fmark;
  __shared__ int s_fail;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gi = tid >> 5, l32 = tid & 31;
  const int B = a.B, d = a.d_model, r = a.r, rc = d - r;
  const int G = gridDim.x, w = blockIdx.x;
  const int n0 = nfirst(w, a.d_ff, G), n1 = nfirst(w + 1, a.d_ff, G), nown = n1 - n0;
  float* qs1 = dyn;
  float* qs2 = dyn + (size_t)BM * r;
  if (tid == 0) {
    const uint32_t t0 = (uint32_t)get_word(hdr);
    s_tag = t0 + 1;
    // one failure mark per call (each layer of it advances the tag by one),
    // so a call counts once however many of its layers time out
    s_fmark = (uint64_t)(t0 + 1 - (uint32_t)layer);
    // hdr[3], when nonzero, is the host-set test hook: it bounds every wait
    // and makes the exchange wait for a tag no word carries
    const uint64_t lim = get_word(hdr + 3);
    s_spin = lim ? (uint32_t)lim : (1u << 22);
    s_poison = lim ? 0x80000000u : 0u;
    // an earlier layer of this call failed (that launch ended before this
    // one began, so every workgroup reads the same): this layer fails too
    s_fail = get_word(hdr + 1) == s_fmark ? 1 : 0;
  }
  // ---------------- the scores.  The small loads first (the previous layer's
  // sums of squares, q[:r] of every token: one 16-byte piece per thread and
  // token, r <= 4 kBThreads), then the K1 fragments, so that waiting for the
  // small ones does not wait for the fragments.
  const bool pre = a.prenorm && gi < B;
  float ssv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int g3 = l32 + 32 * k;
    ssv[k] = pre && g3 < a.G3 ? a.ssp[(size_t)g3 * BM + gi] : 0.f;
  }
  const bool qin = 4 * tid < r;
  f32x4 xq[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b)
    xq[b] = b < B && qin ? *reinterpret_cast<const f32x4*>(a.yin + (size_t)b * d + 4 * tid) : f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 fa[kMTiles][kMSteps];
  {
    int row[kMTiles];
    bool want[kMTiles];
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) {
      row[t] = min(n0 + 16 * t + (lane & 15), n1 - 1);
      want[t] = true;
    }
    mfma_rows_load<NW>(fa, (const char*)a.k1t, (size_t)r * sizeof(bf16_t), row, want, r / 32, wv, lane);
  }
  // each token's RMS scale (half-wave b, fixed order)
  if (gi < BM) {
    float sc = 1.f;
    if (pre) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) ss += ssv[k];
      for (int g3 = l32 + 256; g3 < a.G3; g3 += 32) ss += a.ssp[(size_t)g3 * BM + gi];  // more than 256 segments
      ss = half_sum(ss);
      sc = 1.f / sqrtf(ss / (float)d + a.eps);
    }
    if (l32 == 0) red[gi] = sc;
  }
  // q[:r] unscaled (the scale goes on the sums); empty token slots zero
  if (qin) {
#pragma unroll
    for (int b = 0; b < BM; ++b) *reinterpret_cast<f32x4*>(qs1 + (size_t)b * r + 4 * tid) = xq[b];
  }
  __syncthreads();
  if (s_fail) {
    bfused_failed<BM>(a, hdr, n0, nown, s_tag);
    return;
  }
  if (w == 0 && tid < B) a.scale[tid] = red[tid];
  mfma_rows_products<BM, NW>(fa, qs1, r, r / 32, part, wv, lane);
  __syncthreads();
  for (int i = tid; i < BM * kBSlots; i += kBThreads) {
    const int b = i / kBSlots, j = i % kBSlots;
    if (b < B && j < nown) {
      const float h = mfma_rows_sum<NW>(part, j, b) * red[b];
      hs[b][j] = h;
      a.H[(size_t)b * a.d_ff + n0 + j] = h;
    }
  }
  __syncthreads();
  // ---------------- this workgroup's (mean, M2) per token, published
  const uint32_t tag = s_tag;
  for (int b = wv; b < B; b += NW) {
    const bool own = lane < nown;
    const float h = own ? hs[b][lane] : 0.f;
    const float mean = wave_sum_dpp(h) / (float)nown;
    const float dv = own ? h - mean : 0.f;
    const float m2 = wave_sum_dpp(dv * dv);
    if (lane < kXRep) {
      uint64_t* dst = xs + (size_t)lane * xs_stride + (size_t)(2 * b) * kXRow + w;
      put_tagged(dst, mean, tag);
      put_tagged(dst + kXRow, m2, tag);
    }
  }
  // q[r:] of every token, scaled (used after the exchange; the barrier after
  // it orders these LDS writes before the K2 products)
  {
    const bool kin = 4 * tid < rc;
    f32x4 xk[BM];
#pragma unroll
    for (int b = 0; b < BM; ++b)
      xk[b] = b < B && kin ? *reinterpret_cast<const f32x4*>(a.yin + (size_t)b * d + r + 4 * tid)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
    if (kin) {
#pragma unroll
      for (int b = 0; b < BM; ++b) *reinterpret_cast<f32x4*>(qs2 + (size_t)b * rc + 4 * tid) = xk[b] * red[b];
    }
  }
  // ---------------- every workgroup's (mean, M2) of token gi (half-wave gi,
  // workgroups l32 + 32 k), then theta (the mean, then the squared deviations
  // about it, fixed order)
  if (gi < B) {
    const int b = gi;
    const uint64_t* src = xs + (size_t)xcc_id() * xs_stride + (size_t)(2 * b) * kXRow;
    constexpr int KG = 8;  // G <= 256
    float mn[KG], m2v[KG], nn[KG];
    uint32_t need = 0;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int g = l32 + 32 * k;
      need |= g < G ? 3u << (2 * k) : 0u;
      nn[k] = g < G ? (float)(nfirst(g + 1, a.d_ff, G) - nfirst(g, a.d_ff, G)) : 0.f;
      mn[k] = m2v[k] = 0.f;
    }
    const uint32_t want_tag = tag ^ s_poison, spin_limit = s_spin;
    bool ok = true;
    for (uint32_t spin = 0; need; ++spin) {
      uint64_t x[2 * KG];
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          x[2 * k + q] = ((need >> (2 * k + q)) & 1) ? get_word(src + (size_t)q * kXRow + l32 + 32 * k) : 0;
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (((need >> (2 * k + q)) & 1) && (uint32_t)(x[2 * k + q] >> 32) == want_tag) {
            const float v = __uint_as_float((uint32_t)x[2 * k + q]);
            if (q == 0)
              mn[k] = v;
            else
              m2v[k] = v;
            need &= ~(1u << (2 * k + q));
          }
      if (!need) break;
      if (spin > spin_limit || ((spin & 1023) == 1023 && get_word(hdr + 1) == s_fmark)) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    float s1 = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) s1 += nn[k] * mn[k];
    const float mu = half_sum(s1) / (float)a.d_ff;
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const float dm = mn[k] - mu;
      s2 += nn[k] > 0.f ? m2v[k] + nn[k] * dm * dm : 0.f;
    }
    s2 = half_sum(s2);
    if (l32 == 0) th[b] = mu + sqrtf(s2 / (float)a.d_ff) * a.z;
    if (!ok) {
      s_fail = 1;
      raise_failure(hdr, s_fmark);
    }
  }
  __syncthreads();
  if (s_fail) {
    bfused_failed<BM>(a, hdr, n0, nown, tag);
    return;
  }
  if (w == 0 && tid < B) a.theta[tid] = th[tid];
  // ---------------- the tokens selecting each owned neuron
  if (tid < kBSlots) {
    uint32_t m = 0;
    for (int b = 0; b < B; ++b) m |= (tid < nown && hs[b][tid] > th[b]) ? 1u << b : 0u;
    sel[tid] = m;
  }
  __syncthreads();
  // ---------------- the K2 dots of the selected neurons on the matrix cores
  {
    int row[kMTiles];
    bool want[kMTiles];
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) {
      const int j = 16 * t + (lane & 15);
      row[t] = min(n0 + j, n1 - 1);
      want[t] = j < nown && j < kBSlots && sel[j < kBSlots ? j : 0] != 0;
    }
    mfma_rows_load<NW>(fa, (const char*)a.k2t, (size_t)rc * sizeof(bf16_t), row, want, rc / 32, wv, lane);
    mfma_rows_products<BM, NW>(fa, qs2, rc, rc / 32, part, wv, lane);
  }
  __syncthreads();
  for (int i = tid; i < BM * kBSlots; i += kBThreads) {
    const int b = i / kBSlots, j = i % kBSlots;
    if (b < B && j < nown) {
      const bool on = (sel[j] >> b) & 1u;
      const float g = mfma_rows_sum<NW>(part, j, b);
      a.C[(size_t)(n0 + j) * BM + b] = on ? gelu_tanh(hs[b][j] - th[b]) * g : 0.f;
    }
  }
  if (tid < 64) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(lane < kBSlots && sel[lane < kBSlots ? lane : 0] != 0);
    if (lane == 0) a.umask[w] = m;
  }
  // every workgroup has read the header before publishing, and workgroup 0
  // gets here only after every workgroup published
  if (w == 0 && tid == 0) __hip_atomic_store(hdr, (uint64_t)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct BatchLayout {
  size_t H, P, scale, theta, umask, C, ybuf, ssp, P2, X, X2, total;
  int xs_stride;  // words between the exchange replicas of bfused
};

// Workgroups of bpred and bgate: one per CU, more when a CU's share of the
// neurons would exceed kBSlots, fewer when it would fall below 4.
static int batch_groups(int64_t d_ff) {
  int64_t G = device_cu_count();
  if (G < 1) G = 256;
  if (G > d_ff / 4) G = d_ff / 4 > 0 ? d_ff / 4 : 1;
  if ((d_ff + G - 1) / G > kBSlots) G = (d_ff + kBSlots - 1) / kBSlots;
  return (int)G;
}

// bv2 workgroups (column blocks x slices) whose slice sums the folded
// reduction can hold: about two per CU plus one block's worth of rounding
// (bfused shapes have d_model <= 2 x 1280, at most 40 column blocks).  The
// area is sized without B or d_model, so it sits at the same place for every
// call on a workspace and holds only tagged words.
static int fold_blocks_cap() {
  int cus = device_cu_count();
  if (cus < 1) cus = 256;
  return 2 * cus + 64;
}

static BatchLayout batch_layout(int64_t d_model, int64_t d_ff, int64_t B) {
  const int64_t G = batch_groups(d_ff);
  BatchLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, 256);
    return o;
  };
  // the tagged exchange words first: their place does not depend on B, so
  // calls with any batch size on one workspace only ever leave tagged words
  // (or zeros) there
  L.xs_stride = (int)round_up((size_t)2 * kBatchMax * kXRow + 64, 512);  // replicas 4 KB+ apart
  L.X = take((size_t)kXRep * L.xs_stride * 8);
  L.X2 = take((size_t)fold_blocks_cap() * kBatchMax * kFoldCols * 8);
  L.H = take((size_t)B * d_ff * 4);
  L.P = take((size_t)G * B * 2 * 4);
  L.scale = take((size_t)B * 4);
  L.theta = take((size_t)B * 4);
  L.umask = take((size_t)G * 8);
  L.C = take((size_t)d_ff * kBatchMax * 4);
  L.ybuf = take((size_t)B * d_model * 4);
  L.ssp = take((size_t)8192 * kBatchMax * 4);  // reduce workgroups (at most 8192) x token slots
  // bv2's slices x tokens x columns, for more than one token (bf16's wider
  // chunks make fewer column blocks, hence more slices)
  const int s4 = bv2_slices(d_model, 4), s8 = bv2_slices(d_model, 8);
  const int64_t S = B <= 1 ? 0 : (s4 > s8 ? s4 : s8);
  L.P2 = take((size_t)S * B * d_model * 4);
  L.total = off;
  return L;
}

size_t decode_batched_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t B) {
  return batch_layout(d_model, d_ff, B).total;
}


template <typename W, int BM>
static hipError_t launch_batched_t(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                   const float* q, int64_t B, float* y, float eps, double z,
                                   const spark_ffn_trace* trace, void* ws, uint64_t* hdr, hipStream_t st) {
  constexpr int CN = Chunk<W>::N;
  const BatchLayout Lo = batch_layout(s.d_model, s.d_ff, B);
  char* base = (char*)ws;
  const int G = batch_groups(s.d_ff);
  const int nchunks = (int)(s.d_model / CN);
  // one token: bv, each workgroup one or two 16-byte output chunks;
  // more: bv2 by (128-byte column block, union slice), then breduce by
  // 256-column segment.  G3 counts the workgroups that leave a sum of
  // squares per token.
  constexpr bool kSmall = BM <= 1;
  const int nblocks = (nchunks + 7) / 8;      // bv2 column blocks (128-byte lines)
  const int S = bv2_slices(s.d_model, CN);    // bv2 union slices per block
  // both products on the matrix cores in one kernel per layer, when the device
  // holds the whole grid at once (its workgroups exchange the statistics
  // while they run)
  constexpr int kMaxK = 32 * kMSteps * (kBThreads / 64);
  const bool mf1 = kMatrixOk<W> && s.r % 32 == 0 && s.r <= kMaxK;
  bool fused = false;
  const size_t ldsf = (size_t)BM * s.d_model * 4;
  if (kMatrixOk<W> && mf1 && (s.d_model - s.r) % 32 == 0 && s.d_model - s.r <= kMaxK && G <= kXRow) {
    int per_cu = 0;
    if (hipFuncSetAttribute((const void*)bfused<BM>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsf) ==
            hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bfused<BM>, kBThreads, ldsf) == hipSuccess &&
        (int64_t)per_cu * device_cu_count() >= G)
      fused = true;
    (void)hipGetLastError();
  }
  // with bfused (which advances the header's tag every layer) and two or more
  // tokens, bv2 reduces its slices itself: no breduce launch
  const bool fold = !kSmall && fused && 8 * CN == kFoldCols && nblocks * S <= fold_blocks_cap();
  int G3;
  if (fold) {
    G3 = nblocks;
  } else if (kSmall) {
    G3 = device_cu_count();
    if (G3 < 1) G3 = 256;
    if (G3 > nchunks) G3 = nchunks;
    if (2 * G3 < nchunks) G3 = (nchunks + 1) / 2;
  } else {
    G3 = (int)((s.d_model + kRedCols - 1) / kRedCols);
  }
  // (BM token slots; the entry point keeps BM x max(r, d - r) x 4 within
  // kBatchMaxLds)
  const size_t lds1 = (size_t)BM * s.r * 4, lds2 = (size_t)BM * (s.d_model - s.r) * 4;
  hipError_t e = hipSuccess;
  BatchArgs a;
  a.G3 = G3;
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
  a.umask = (uint64_t*)(base + Lo.umask);
  a.C = (float*)(base + Lo.C);
  a.ssp = (float*)(base + Lo.ssp);
  float* ybuf = (float*)(base + Lo.ybuf);
  // the predictor and K2 products on the matrix cores where the shapes allow
  // (the K2 dots: at eight token slots; with fewer, the extra barrier and the
  // full-tile loads of the matrix-core form cost more than the vector units'
  // products, measured)
  const bool mf2 = kMatrixOk<W> && BM >= 8 && (s.d_model - s.r) % 32 == 0 && s.d_model - s.r <= kMaxK;
  for (int l = 0; l < n_layers; ++l) {
    a.k1t = layers[l].k1t;
    a.k2t = layers[l].k2t;
    a.v = layers[l].v;
    a.yin = l == 0 ? q : ybuf;
    a.prenorm = l == 0 ? 0 : 1;
    a.yout = l == n_layers - 1 ? y : ybuf;
    if (fused) {
      hipLaunchKernelGGL((bfused<BM>), dim3(G), dim3(kBThreads), ldsf, st, a, hdr, (uint64_t*)(base + Lo.X),
                         Lo.xs_stride, l);
    } else {
      if (mf1)
        hipLaunchKernelGGL((bpred<W, BM, kMatrixOk<W>>), dim3(G), dim3(kBThreads), lds1, st, a);
      else
        hipLaunchKernelGGL((bpred<W, BM, false>), dim3(G), dim3(kBThreads), lds1, st, a);
      if (mf2)
        hipLaunchKernelGGL((bgate<W, BM, kMatrixOk<W> && BM >= 8>), dim3(G), dim3(kBThreads), lds2, st, a);
      else
        hipLaunchKernelGGL((bgate<W, BM, false>), dim3(G), dim3(kBThreads), lds2, st, a);
    }
    if (trace && (trace->counts || trace->idx || trace->theta || trace->q_in))
      hipLaunchKernelGGL(btrace, dim3((unsigned)B), dim3(256), 0, st, a, trace->counts, trace->idx,
                         trace->idx ? trace->cap : 0, trace->theta, trace->q_in, (int64_t)l, (int64_t)n_layers);
    // bv (or breduce) overwrites ybuf (the input of this layer) only after
    // bpred, bgate and the trace have read it: they precede it on the stream
    if constexpr (kSmall) {
      hipLaunchKernelGGL((bv<W, BM>), dim3(G3), dim3(kBvThreads), 0, st, a, G);
    } else {
      bool folded = false;
      if constexpr (kMatrixOk<W>) {
        if (fold) {
          hipLaunchKernelGGL((bv2<W, BM, true>), dim3((unsigned)(nblocks * S)), dim3(kBv2Threads), 0, st, a, G, S,
                             (float*)nullptr, hdr, (uint64_t*)(base + Lo.X2), l);
          folded = true;
        }
      }
      if (!folded) {
        hipLaunchKernelGGL((bv2<W, BM, false>), dim3((unsigned)(nblocks * S)), dim3(kBv2Threads), 0, st, a, G, S,
                           (float*)(base + Lo.P2), (uint64_t*)nullptr, (uint64_t*)nullptr, l);
        hipLaunchKernelGGL((breduce<BM>), dim3((unsigned)G3, (unsigned)B), dim3(64), 0, st, a, S,
                           (const float*)(base + Lo.P2));
      }
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename W>
static hipError_t launch_batched_w(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                   const float* q, int64_t B, float* y, float eps, double z,
                                   const spark_ffn_trace* trace, void* ws, uint64_t* hdr, hipStream_t st) {
  if (B <= 1) return launch_batched_t<W, 1>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
  if (B <= 2) return launch_batched_t<W, 2>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
  if (B <= 4) return launch_batched_t<W, 4>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
  return launch_batched_t<W, 8>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
}

hipError_t launch_decode_batched(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                 const float* q, int64_t B, float* y, float eps, double z,
                                 const spark_ffn_trace* trace, void* ws, uint64_t* hdr, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (s.wdtype == SPARK_BF16)
    return launch_batched_w<bf16_t>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
  return launch_batched_w<float>(s, layers, n_layers, q, B, y, eps, z, trace, ws, hdr, st);
}

}  // namespace spark
