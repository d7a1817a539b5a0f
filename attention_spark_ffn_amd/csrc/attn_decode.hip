// Spark attention, one decode step.
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", item
// "Spark Attention"): attention written in the form of the Spark FFN; the key
// dimension is split into a predictor part (first r dims) and a compute part,
// sigma1 = softmax over the statistically top-k'd predictor scores (about
// k_attn tokens attended), sigma2 = softplus of the compute-part scores.  Per
// query head h with KV head g = h / (Hq/Hkv):
//   s_j = q_h[:r] . k1[g][j];  S = stat top-k of s (all j when n_ctx <= k_attn)
//   out_h = sum_{j in S} softmax_S(s)_j * softplus(q_h[r:] . k2[g][j]) * v[g][j]
//
// gfx950 mapping:
//   attn_scores: the predictor scan, the only pass over all n_ctx tokens.  A
//     workgroup takes 256 tokens of one KV head; 16 lanes read one 16-byte
//     chunk each of a token's k1 row (r = 128 bf16 is exactly one 256-byte
//     row per 16 lanes), multiply by both (all) query heads of the group held
//     in registers, and reduce within the 16-lane DPP row.
//   attn_select_gather: one 1024-thread workgroup per query head: mean and
//     squared deviations of the scores (two exact passes), theta, ascending
//     compaction of the selected tokens (one block scan over per-thread
//     contiguous segments), softmax over S, softplus gates from the k2 rows,
//     and the weighted sum of the v rows, every reduction in a fixed order.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kScoreTokens = 256;  // tokens per score workgroup (16 passes of 16)
constexpr int kMaxGroup = 8;       // query heads per KV head handled in registers

__global__ __launch_bounds__(256) void attn_scores(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k1,
                                                   int Hq, int Hkv, int n_ctx, int hd, int r,
                                                   float* __restrict__ scores) {
  const int tid = threadIdx.x, l16 = tid & 15, tok = tid >> 4;  // 16 tokens per pass
  const int group = Hq / Hkv;
  const int nsplit = (n_ctx + kScoreTokens - 1) / kScoreTokens;
  const int g = blockIdx.x / nsplit, j0 = (blockIdx.x % nsplit) * kScoreTokens;
  const int CT = r / 8;  // 16-byte chunks per k1 row
  for (int h0 = 0; h0 < group; h0 += kMaxGroup) {
    const int nh = min(kMaxGroup, group - h0);
    for (int cb = 0; cb < CT; cb += 16) {
      const int c = cb + l16;
      // this lane's q chunk for each head of the group
      float qv[kMaxGroup][8];
#pragma unroll
      for (int u = 0; u < kMaxGroup; ++u) {
        const int h = g * group + h0 + min(u, nh - 1);
        float wf[8];
        Chunk<bf16_t>::widen(load16(q + (size_t)h * hd + (size_t)min(c, CT - 1) * 8), wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[u][e] = (c < CT && u < nh) ? wf[e] : 0.f;
      }
      for (int p = 0; p < kScoreTokens / 16; p += 4) {
        u32x4 raw[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int j = min(j0 + (p + pp) * 16 + tok, n_ctx - 1);
          raw[pp] = load16(k1 + ((size_t)g * n_ctx + j) * r + (size_t)min(c, CT - 1) * 8);
        }
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int j = j0 + (p + pp) * 16 + tok;
          float wf[8];
          Chunk<bf16_t>::widen(raw[pp], wf);
#pragma unroll
          for (int u = 0; u < kMaxGroup; ++u) {
            if (u < nh) {
              float a = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) a += wf[e] * qv[u][e];
              a = row16_sum(a);
              if (l16 == 0 && j < n_ctx) {
                float* dst = scores + (size_t)(g * group + h0 + u) * n_ctx + j;
                *dst = cb == 0 ? a : *dst + a;
              }
            }
          }
        }
      }
    }
  }
}

// Fixed-order reductions over the 1024 threads of the selection kernel.
struct SelShared {
  float red[16];
  int ired[16];
  int wpre[16];
};
__device__ __forceinline__ float block_sum(float v, SelShared& S) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_sum_dpp(v);
  __syncthreads();
  if (lane == 0) S.red[wv] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) t += S.red[w];
  return t;
}
__device__ __forceinline__ float block_max(float v, SelShared& S) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) S.red[wv] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int w = 0; w < 16; ++w) t = fmaxf(t, S.red[w]);
  return t;
}

__global__ __launch_bounds__(1024) void attn_select_gather(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k2, const bf16_t* __restrict__ v, int Hq, int Hkv,
    int n_ctx, int hd, int r, int dense, float z, const float* __restrict__ scores, int32_t* __restrict__ lidx,
    float* __restrict__ lval, float* __restrict__ out, int32_t* __restrict__ counts, int32_t* __restrict__ idx_out,
    int64_t cap, float* __restrict__ theta_out) {
  __shared__ SelShared S;
  __shared__ alignas(16) float qc[512];    // q_h[r:]
  __shared__ float opart[4][512];          // per-quarter sums of the output
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = h / (Hq / Hkv), rc = hd - r;
  const float* s = scores + (size_t)h * n_ctx;
  int32_t* li = lidx + (size_t)h * n_ctx;
  float* lv = lval + (size_t)h * n_ctx;
  for (int c = tid; c < rc; c += 1024) qc[c] = bf16_to_f32(q[(size_t)h * hd + r + c]);
  // thread-contiguous segment of the scores
  const int seg = (n_ctx + 1023) / 1024, a0 = min(tid * seg, n_ctx), a1 = min(a0 + seg, n_ctx);
  float theta = NAN;
  if (!dense) {
    float t1 = 0.f;
    for (int j = a0; j < a1; ++j) t1 += s[j];
    const float mean = block_sum(t1, S) / (float)n_ctx;
    float t2 = 0.f;
    for (int j = a0; j < a1; ++j) {
      const float d = s[j] - mean;
      t2 += d * d;
    }
    const float m2 = block_sum(t2, S);
    theta = mean + sqrtf(m2 / (float)n_ctx) * z;
  }
  // ascending compaction of the selected tokens
  int cnt = 0;
  float smax = -INFINITY;
  for (int j = a0; j < a1; ++j) {
    const bool on = dense || s[j] > theta;
    cnt += on ? 1 : 0;
    smax = on ? fmaxf(smax, s[j]) : smax;
  }
  const int pre_w = wave_excl_scan(cnt, lane);
  const int wtot = __shfl(pre_w + cnt, 63, 64);
  __syncthreads();
  if (lane == 0) S.ired[wv] = wtot;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    base += w < wv ? S.ired[w] : 0;
    total += S.ired[w];
  }
  int pos = base + pre_w;
  for (int j = a0; j < a1; ++j) {
    if (dense || s[j] > theta) {
      li[pos] = j;
      lv[pos] = s[j];
      ++pos;
    }
  }
  const float mx = block_max(smax, S);
  __syncthreads();  // list entries written by other threads
  // softmax denominator over S (ascending order within each thread's slice)
  const int per = (total + 1023) / 1024, b0 = min(tid * per, total), b1 = min(b0 + per, total);
  float den = 0.f;
  for (int e = b0; e < b1; ++e) den += __expf(lv[e] - mx);
  den = block_sum(den, S);
  // gates: softplus(q[r:] . k2[g][j]) for every selected token; 16 lanes per token
  const int CT2 = rc / 8, l16 = lane & 15, sub = tid >> 4;  // 64 tokens per pass
  for (int e0 = 0; e0 < total; e0 += 64) {
    const int e = e0 + sub;
    const int j = li[min(e, total - 1)];
    float acc = 0.f;
    for (int cb = 0; cb < CT2; cb += 16) {
      const int c = cb + l16;
      float wf[8];
      Chunk<bf16_t>::widen(load16(k2 + ((size_t)g * n_ctx + j) * rc + (size_t)min(c, CT2 - 1) * 8), wf);
      const float* qq = qc + min(c, CT2 - 1) * 8;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a += wf[i] * qq[i];
      acc += c < CT2 ? a : 0.f;
    }
    acc = row16_sum(acc);
    __syncthreads();  // every lane has read lv[e] before it is overwritten below
    if (l16 == 0 && e < total) lv[e] = (__expf(lv[e] - mx) / den) * softplus(acc);
  }
  __syncthreads();
  // out[c] = sum over S (ascending, in four interleaved quarters) of w u v[c]
  const int c = tid & 255, quarter = tid >> 8;
  float o = 0.f;
  if (c < hd)
    for (int e = quarter; e < total; e += 4) {
      const int j = li[e];
      o += lv[e] * bf16_to_f32(v[((size_t)g * n_ctx + j) * hd + c]);
    }
  if (c < hd) opart[quarter][c] = o;
  __syncthreads();
  if (tid < hd) out[(size_t)h * hd + tid] = ((opart[0][tid] + opart[1][tid]) + opart[2][tid]) + opart[3][tid];
  if (hd > 256)  // wider heads: the remaining columns, same order
    for (int cc = 256 + tid; cc < hd; cc += 1024) {
      float oo = 0.f;
      for (int e = 0; e < total; ++e) oo += lv[e] * bf16_to_f32(v[((size_t)g * n_ctx + li[e]) * hd + cc]);
      out[(size_t)h * hd + cc] = oo;
    }
  if (tid == 0) {
    if (counts) counts[h] = total;
    if (theta_out) theta_out[h] = theta;
  }
  if (idx_out)
    for (int e = tid; e < cap; e += 1024) idx_out[(size_t)h * cap + e] = e < total ? li[e] : -1;
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t attn_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn) {
  (void)Hkv, (void)hd, (void)r, (void)k_attn;
  return 3 * round_up((size_t)Hq * n_ctx * 4, 256);
}

hipError_t launch_attn_decode(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq, int64_t Hkv,
                              int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double z, float* out,
                              int32_t* counts, int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st) {
  char* base = (char*)ws;
  const size_t plane = round_up((size_t)Hq * n_ctx * 4, 256);
  float* scores = (float*)base;
  int32_t* lidx = (int32_t*)(base + plane);
  float* lval = (float*)(base + 2 * plane);
  const int nsplit = (int)((n_ctx + kScoreTokens - 1) / kScoreTokens);
  hipLaunchKernelGGL(attn_scores, dim3((unsigned)(Hkv * nsplit)), dim3(256), 0, st, (const bf16_t*)q,
                     (const bf16_t*)k1, (int)Hq, (int)Hkv, (int)n_ctx, (int)hd, (int)r, scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int dense = n_ctx <= k_attn ? 1 : 0;
  hipLaunchKernelGGL(attn_select_gather, dim3((unsigned)Hq), dim3(1024), 0, st, (const bf16_t*)q, (const bf16_t*)k2,
                     (const bf16_t*)v, (int)Hq, (int)Hkv, (int)n_ctx, (int)hd, (int)r, dense, (float)z, scores, lidx,
                     lval, out, counts, idx, cap, theta);
  return hipGetLastError();
}

}  // namespace spark
