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
// gfx950 mapping: the context is cut into chunks of CK tokens (64, 128 or 256:
// the largest that still gives the scan at least 256 workgroups), and every
// step runs over (head, chunk) pairs so that the whole chip works on one
// decode step:
//   attn_scores (KV head, chunk): the predictor scan, the only pass over all
//     n_ctx tokens.  16 lanes read one 16-byte chunk each of a token's k1 row
//     (r = 128 bf16 is one 256-byte row per 16 lanes), all 16 tokens of a
//     lane group's rows are loaded before any is used, and every query head of
//     the group is applied from registers (DPP row sums).  The workgroup also
//     writes each head's (mean, M2) over the chunk.
//   attn_chunk (query head, chunk): theta from the chunk statistics (the same
//     fixed-order combination in every workgroup of the head), the chunk's
//     selected tokens in ascending order, their softplus gates from the k2
//     rows, and the chunk's part of the softmax-weighted sum of v rows relative
//     to the chunk's own maximum score (m_c, l_c = sum of e^(s - m_c), o_c).
//   attn_merge (query head): out = sum_c e^(m_c - m) o_c / sum_c e^(m_c - m) l_c
//     with m the largest m_c, the count, theta and (when asked for) the
//     ascending list.  Every sum runs in a fixed order.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kMaxGroup = 8;      // query heads per KV head handled in registers
constexpr int kMaxChunks = 4096;  // chunks per head (n_ctx <= 2^20)

// Chunk length of a context: 64, 128 or 256 tokens, the largest giving the
// scan at least 256 workgroups.  A shorter chunk is only taken while n_ctx <
// 256 * 128, so a head never has more than kMaxChunks chunks for n_ctx <=
// 2^20 (the interface's limit).  The workspace layout and the launch both
// take the length from here.
static int chunk_tokens(int64_t Hkv, int64_t n_ctx) {
  int ck = 256;
  while (ck > 64 && Hkv * ((n_ctx + ck - 1) / ck) < 256) ck >>= 1;
  return ck;
}

template <int kChunk>
__global__ __launch_bounds__(256) void attn_scores(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k1,
                                                   int Hq, int Hkv, int n_ctx, int hd, int r,
                                                   float* __restrict__ scores, float2* __restrict__ cstat) {
  __shared__ float sc[kMaxGroup][kChunk];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = tid & 15, tok = tid >> 4;  // 16 tokens/pass
  const int group = Hq / Hkv;
  const int nch = (n_ctx + kChunk - 1) / kChunk;
  const int g = blockIdx.x / nch, c0 = blockIdx.x % nch, j0 = c0 * kChunk;
  const int nc = min(kChunk, n_ctx - j0);
  const int CT = r / 8;  // 16-byte chunks per k1 row
  for (int h0 = 0; h0 < group; h0 += kMaxGroup) {
    const int nh = min(kMaxGroup, group - h0);
    for (int cb = 0; cb < CT; cb += 16) {
      const int c = cb + l16;
      // every k1 load of the lane first (16 tokens), then the q chunks
      u32x4 raw[kChunk / 16];
#pragma unroll
      for (int p = 0; p < kChunk / 16; ++p) {
        const int j = min(j0 + p * 16 + tok, n_ctx - 1);
        raw[p] = load16(k1 + ((size_t)g * n_ctx + j) * r + (size_t)min(c, CT - 1) * 8);
      }
      float qv[kMaxGroup][8];
#pragma unroll
      for (int u = 0; u < kMaxGroup; ++u) {
        const int h = g * group + h0 + min(u, nh - 1);
        float wf[8];
        Chunk<bf16_t>::widen(load16(q + (size_t)h * hd + (size_t)min(c, CT - 1) * 8), wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[u][e] = (c < CT && u < nh) ? wf[e] : 0.f;
      }
#pragma unroll
      for (int p = 0; p < kChunk / 16; ++p) {
        const int t = p * 16 + tok;
        float wf[8];
        Chunk<bf16_t>::widen(raw[p], wf);
#pragma unroll
        for (int u = 0; u < kMaxGroup; ++u) {
          if (u < nh) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a += wf[e] * qv[u][e];
            a = row16_sum(a);
            if (l16 == 0) sc[u][t] = cb == 0 ? a : sc[u][t] + a;
          }
        }
      }
    }
    __syncthreads();
    // scores out, and each head's (mean, M2) over the chunk: wave w takes heads
    // w, w + 4, each lane four tokens
    for (int e = tid; e < nh * kChunk; e += 256) {
      const int u = e / kChunk, t = e % kChunk;
      if (t < nc) scores[(size_t)(g * group + h0 + u) * n_ctx + j0 + t] = sc[u][t];
    }
    for (int u = wv; u < nh; u += 4) {
      float x[kChunk / 64], s1 = 0.f;
#pragma unroll
      for (int i = 0; i < kChunk / 64; ++i) {
        const int t = lane + 64 * i;
        x[i] = t < nc ? sc[u][t] : 0.f;
        s1 += x[i];
      }
      const float mean = wave_sum_dpp(s1) / (float)nc;
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < kChunk / 64; ++i) {
        const float d = x[i] - mean;
        s2 += lane + 64 * i < nc ? d * d : 0.f;
      }
      const float m2 = wave_sum_dpp(s2);
      if (lane == 0) cstat[(size_t)(g * group + h0 + u) * nch + c0] = make_float2(mean, m2);
    }
    __syncthreads();
  }
}

// Fixed-order reductions over the 256 threads of a chunk workgroup.
__device__ __forceinline__ float block_max256(float v, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

// theta of head h from its chunk statistics: mean = sum n_c mean_c / n, then
// M2 = sum (M2_c + n_c (mean_c - mean)^2) (two plain sums in a fixed order,
// Chan et al.'s combination).  Called by one wave; every lane gets the result.
template <int kChunk>
__device__ __forceinline__ float head_theta(const float2* __restrict__ cst, int nch, int n_ctx, float z, int lane) {
  float s1 = 0.f;
  for (int c = lane; c < nch; c += 64) s1 += (float)min(kChunk, n_ctx - c * kChunk) * cst[c].x;
  const float mean = wave_sum_dpp(s1) / (float)n_ctx;
  float s2 = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const float2 st = cst[c];
    const float d = st.x - mean;
    s2 += st.y + (float)min(kChunk, n_ctx - c * kChunk) * d * d;
  }
  const float m2 = wave_sum_dpp(s2);
  return mean + sqrtf(m2 / (float)n_ctx) * z;
}

// Partial of one (query head, chunk): m_c, l_c, count, then o_c[hd].
constexpr int kPartHead = 4;

template <int kChunk>
__global__ __launch_bounds__(256) void attn_chunk(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k2,
                                                  const bf16_t* __restrict__ v, int Hq, int Hkv, int n_ctx, int hd,
                                                  int r, int dense, float z, const float* __restrict__ scores,
                                                  const float2* __restrict__ cstat, float* __restrict__ part,
                                                  int32_t* __restrict__ lidx) {
  __shared__ alignas(16) float qc[512];  // q_h[r:]
  __shared__ int loc[kChunk];            // selected tokens of the chunk (offsets), ascending
  __shared__ float sv[kChunk];           // their scores, then e^(s - m_c)
  __shared__ float wu[kChunk];           // e^(s - m_c) * softplus gate
  __shared__ float red[4];
  __shared__ int wcnt[4];
  __shared__ float th_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = (n_ctx + kChunk - 1) / kChunk;
  const int h = blockIdx.x / nch, c0 = blockIdx.x % nch, j0 = c0 * kChunk;
  const int nc = min(kChunk, n_ctx - j0);
  const int g = h / (Hq / Hkv), rc = hd - r;
  for (int c = tid; c < rc; c += 256) qc[c] = bf16_to_f32(q[(size_t)h * hd + r + c]);
  if (wv == 0) {
    const float th = dense ? -INFINITY : head_theta<kChunk>(cstat + (size_t)h * nch, nch, n_ctx, z, lane);
    if (lane == 0) th_s = th;
  }
  const float s = tid < nc ? scores[(size_t)h * n_ctx + j0 + tid] : -INFINITY;
  __syncthreads();
  const float theta = th_s;
  const bool on = tid < nc && (dense || s > theta);
  // ascending compaction within the chunk
  const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
  const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane == 0) wcnt[wv] = __builtin_popcountll(bal);
  __syncthreads();
  int base = 0, cnt = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wv ? wcnt[w] : 0;
    cnt += wcnt[w];
  }
  if (on) {
    loc[base + pre] = tid;
    sv[base + pre] = s;
  }
  const float mc = block_max256(on ? s : -INFINITY, red);  // also orders the list writes
  // gates: softplus(q[r:] . k2[g][j]), 16 lanes per token, 16 tokens per pass
  const int CT2 = rc / 8, l16 = tid & 15, sub = tid >> 4;
  for (int e0 = 0; e0 < cnt; e0 += 16) {
    const int e = e0 + sub;
    const int j = j0 + loc[min(e, cnt - 1)];
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
    if (l16 == 0 && e < cnt) {
      const float p = __expf(sv[e] - mc);
      wu[e] = p * softplus(acc);
      sv[e] = p;
    }
  }
  __syncthreads();
  float* pt = part + (size_t)blockIdx.x * (kPartHead + hd);
  if (tid == 0) {
    float l = 0.f;
    for (int e = 0; e < cnt; ++e) l += sv[e];  // ascending
    pt[0] = mc;
    pt[1] = l;
    pt[2] = __int_as_float(cnt);
    pt[3] = dense ? NAN : theta;  // every token attended: no threshold
  }
  // o_c[col]: sum over the chunk's selected tokens, ascending; four loads in flight
  for (int col = tid; col < hd; col += 256) {
    float o = 0.f;
    int e = 0;
    for (; e + 4 <= cnt; e += 4) {
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = bf16_to_f32(v[((size_t)g * n_ctx + j0 + loc[e + u]) * hd + col]);
#pragma unroll
      for (int u = 0; u < 4; ++u) o += wu[e + u] * x[u];
    }
    for (; e < cnt; ++e) o += wu[e] * bf16_to_f32(v[((size_t)g * n_ctx + j0 + loc[e]) * hd + col]);
    pt[kPartHead + col] = o;
  }
  if (lidx)
    for (int e = tid; e < cnt; e += 256) lidx[(size_t)h * n_ctx + j0 + e] = j0 + loc[e];
}

// One 1024-thread workgroup per query head.  The chunk statistics (m_c, l_c,
// count) are read in one parallel pass; the weighted column sums run in four
// quarters of the chunks (chunk c in quarter c % 4, up to sixteen loads in
// flight per thread) combined in a fixed order.
template <int kChunk>
__global__ __launch_bounds__(1024) void attn_merge(int n_ctx, int hd, const float* __restrict__ part,
                                                   const int32_t* __restrict__ lidx, float* __restrict__ out,
                                                   int32_t* __restrict__ counts, int32_t* __restrict__ idx_out,
                                                   int64_t cap, float* __restrict__ theta_out) {
  __shared__ float wexp[kMaxChunks];  // m_c, then e^(m_c - m)
  __shared__ float lsum[kMaxChunks];  // l_c
  __shared__ int ccnt[kMaxChunks];
  __shared__ float red[16];
  __shared__ int ired[16];
  __shared__ float opart[4][256];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = (n_ctx + kChunk - 1) / kChunk;
  const int stride = kPartHead + hd;
  const float* ph = part + (size_t)h * nch * stride;
  // chunk maxima and counts
  float mx = -INFINITY;
  int cn = 0;
  for (int c = tid; c < nch; c += 1024) {
    const float mc = ph[(size_t)c * stride];
    const float lc = ph[(size_t)c * stride + 1];
    const int k = __float_as_int(ph[(size_t)c * stride + 2]);
    wexp[c] = mc;
    lsum[c] = lc;
    ccnt[c] = k;
    mx = fmaxf(mx, mc);
    cn += k;
  }
  mx = wave_max(mx);
  cn = wave_sum_int(cn);
  if (lane == 0) {
    red[wv] = mx;
    ired[wv] = cn;
  }
  __syncthreads();
  float m = -INFINITY;
  int tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    m = fmaxf(m, red[w]);
    tot += ired[w];
  }
  __syncthreads();
  // weights and the softmax denominator (fixed order: per thread, then lanes, then waves)
  float dsum = 0.f;
  for (int c = tid; c < nch; c += 1024) {
    const float mc = wexp[c];
    const float w = mc == -INFINITY ? 0.f : __expf(mc - m);
    wexp[c] = w;
    dsum += w * lsum[c];
  }
  dsum = wave_sum_dpp(dsum);
  if (lane == 0) red[wv] = dsum;
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) den += red[w];
  // columns
  const int quarter = tid >> 8;
  for (int col0 = 0; col0 < hd; col0 += 256) {
    const int col = col0 + (tid & 255);
    float o = 0.f;
    if (col < hd) {
      int c = quarter;
      for (; c + 60 < nch; c += 64) {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = ph[(size_t)(c + 4 * u) * stride + kPartHead + col];
#pragma unroll
        for (int u = 0; u < 16; ++u) o += wexp[c + 4 * u] * x[u];
      }
      for (; c + 28 < nch; c += 32) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = ph[(size_t)(c + 4 * u) * stride + kPartHead + col];
#pragma unroll
        for (int u = 0; u < 8; ++u) o += wexp[c + 4 * u] * x[u];
      }
      for (; c < nch; c += 4) o += wexp[c] * ph[(size_t)c * stride + kPartHead + col];
    }
    opart[quarter][tid & 255] = o;
    __syncthreads();
    if (tid < 256 && col < hd) {
      const float oo = ((opart[0][tid] + opart[1][tid]) + opart[2][tid]) + opart[3][tid];
      out[(size_t)h * hd + col] = den > 0.f ? oo / den : 0.f;
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (counts) counts[h] = tot;
    if (theta_out) theta_out[h] = ph[3];
  }
  if (idx_out) {  // the ascending list
    // chunk offsets: exclusive prefix of the counts over contiguous segments
    // of chunks (thread-serial), then over threads (block scan)
    const int seg = (nch + 1023) / 1024, a0 = min(tid * seg, nch), a1 = min(a0 + seg, nch);
    int mine = 0;
    for (int c = a0; c < a1; ++c) mine += ccnt[c];
    const int incl = wave_incl_scan_dpp(mine);
    if (lane == 63) ired[wv] = incl;
    __syncthreads();
    int run = incl - mine;
    for (int w = 0; w < wv; ++w) run += ired[w];
    for (int c = a0; c < a1; ++c) {
      const int k = ccnt[c];
      ccnt[c] = run;
      run += k;
    }
    __syncthreads();
    // position p comes from the last chunk whose offset is <= p (binary search)
    const int np = (int)min((int64_t)tot, cap);
    for (int p = tid; p < np; p += 1024) {
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ccnt[mid] <= p) lo = mid; else hi = mid - 1;
      }
      idx_out[(size_t)h * cap + p] = lidx[(size_t)h * n_ctx + lo * kChunk + (p - ccnt[lo])];
    }
    for (int64_t e = tot + tid; e < cap; e += 1024) idx_out[(size_t)h * cap + e] = -1;
  }
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: scores [Hq][n_ctx], chunk statistics [Hq][nch] (mean, M2), chunk
// partials [Hq][nch][4 + hd], chunk-local lists [Hq][n_ctx].
struct AttnLayout {
  size_t scores, cstat, part, lidx, total;
};
static AttnLayout attn_layout(int64_t Hq, int64_t nch, int64_t n_ctx, int64_t hd) {
  AttnLayout L;
  size_t off = 0;
  L.scores = off;
  off += round_up((size_t)Hq * n_ctx * 4, 256);
  L.cstat = off;
  off += round_up((size_t)Hq * nch * 8, 256);
  L.part = off;
  off += round_up((size_t)Hq * nch * (kPartHead + hd) * 4, 256);
  L.lidx = off;
  off += round_up((size_t)Hq * n_ctx * 4, 256);
  L.total = off;
  return L;
}

size_t attn_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn) {
  (void)r, (void)k_attn;
  const int ck = chunk_tokens(Hkv, n_ctx);
  return attn_layout(Hq, (n_ctx + ck - 1) / ck, n_ctx, hd).total;
}

template <int CK>
static hipError_t launch_attn_decode_t(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq,
                                       int64_t Hkv, int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double z,
                                       float* out, int32_t* counts, int32_t* idx, int64_t cap, float* theta, void* ws,
                                       hipStream_t st) {
  const int nch = (int)((n_ctx + CK - 1) / CK);
  const AttnLayout L = attn_layout(Hq, nch, n_ctx, hd);
  char* base = (char*)ws;
  float* scores = (float*)(base + L.scores);
  float2* cstat = (float2*)(base + L.cstat);
  float* part = (float*)(base + L.part);
  int32_t* lidx = idx ? (int32_t*)(base + L.lidx) : nullptr;
  hipLaunchKernelGGL(attn_scores<CK>, dim3((unsigned)(Hkv * nch)), dim3(256), 0, st, (const bf16_t*)q,
                     (const bf16_t*)k1, (int)Hq, (int)Hkv, (int)n_ctx, (int)hd, (int)r, scores, cstat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int dense = n_ctx <= k_attn ? 1 : 0;
  hipLaunchKernelGGL(attn_chunk<CK>, dim3((unsigned)(Hq * nch)), dim3(256), 0, st, (const bf16_t*)q,
                     (const bf16_t*)k2, (const bf16_t*)v, (int)Hq, (int)Hkv, (int)n_ctx, (int)hd, (int)r, dense,
                     (float)z, scores, cstat, part, lidx);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge<CK>, dim3((unsigned)Hq), dim3(1024), 0, st, (int)n_ctx, (int)hd, part, lidx, out,
                     counts, idx, cap, theta);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, const void* k1, const void* k2, const void* v, int64_t Hq, int64_t Hkv,
                              int64_t n_ctx, int64_t hd, int64_t r, int64_t k_attn, double z, float* out,
                              int32_t* counts, int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st) {
  switch (chunk_tokens(Hkv, n_ctx)) {
    case 64:
      return launch_attn_decode_t<64>(q, k1, k2, v, Hq, Hkv, n_ctx, hd, r, k_attn, z, out, counts, idx, cap, theta, ws,
                                      st);
    case 128:
      return launch_attn_decode_t<128>(q, k1, k2, v, Hq, Hkv, n_ctx, hd, r, k_attn, z, out, counts, idx, cap, theta,
                                       ws, st);
    default:
      return launch_attn_decode_t<256>(q, k1, k2, v, Hq, Hkv, n_ctx, hd, r, k_attn, z, out, counts, idx, cap, theta,
                                       ws, st);
  }
}

}  // namespace spark
