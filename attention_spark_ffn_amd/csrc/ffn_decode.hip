// Spark FFN decode: a persistent, cooperative kernel that runs the whole stack of
// layers for each token without returning to the host.
//
// Method (Spark Transformer reading notes, section "方法详解 / 关键设计", item
// "Spark FFN"): y = V (GELU(StatTopk(K1^T q[:r])) (.) (K2^T q[r:])); only the
// selected neurons' K2 columns and V rows are read.  StatTopk is the
// statistical top-k of item "Statistical Top-k".  Between layers
// q <- y / sqrt(mean(y^2) + eps).
//
// Work split (G workgroups, one per CU, 512 threads each):
//   * workgroup w owns the contiguous neuron range [n0, n1) and, for the layer
//     output, the column range [c0, c1);
//   * waves 4..7 ("streamers") hold the workgroup's K1^T slab (rows n0..n1,
//     contiguous in memory) in registers.  Right after a layer's predictor
//     product they issue the loads of the NEXT layer's slab, which then stream
//     from HBM while the rest of the layer runs; they never wait on any other
//     global load, so the barriers of the layer do not wait for the prefetch;
//   * waves 0..3 ("workers") do everything that waits on memory: the
//     statistics exchange, the K2 gather-dot, the V rows, and the exchanges of
//     the layer output.
// Per layer three grid-wide exchanges (A: per-workgroup (mean, M2) of the
// predictor scores -> theta; B: per-workgroup partial y -> column owners;
// C: owned columns of y -> every workgroup) move 64-bit words that carry the
// value and a 32-bit tag.  Writers store them with device-scope relaxed
// atomics (coherent across the eight XCD L2 caches); readers poll until the
// tag of the exchange appears, so no cross-XCD fence is needed.  Exchanges A
// and C are replicated once per XCD so each replica has 32 readers.
// Every wait is bounded: on timeout the kernel records a failure in the
// workspace header and all workgroups leave.
#include "common.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kDecMaxC = 21;  // K1 chunks (16 B) held per streamer thread (a 36 x 1152 bf16 slab)
constexpr int kStreamers = 256;
constexpr int kWorkers = 256;
constexpr int kRep = 8;       // replicas of the broadcast exchanges (one per XCD)
constexpr int kRedMax = kDecodeMaxDModel + 512;

struct DecodeParams {
  const void* k1t[kDecodeMaxLayersPerLaunch];
  const void* k2t[kDecodeMaxLayersPerLaunch];
  const void* v[kDecodeMaxLayersPerLaunch];
  int n_layers, layer_offset, total_layers;
  int d_model, d_ff, r, T;
  float z, eps;
  const float* q_in;
  int q_prenorm;
  float* y_out;
  int32_t* tr_counts;
  int32_t* tr_idx;
  float* tr_theta;
  float* tr_q;
  int64_t tr_cap;
  uint64_t* hdr;   // [0]: last tag used, [1]: failure flag
  uint64_t* stats; // kRep x stats_stride
  uint64_t* part;  // G x part_stride
  uint64_t* ycol;  // kRep x ycol_stride
  int stats_stride, part_stride, ycol_stride;
  uint32_t spin_limit;
};

// Poll up to K tagged words (a null pointer is skipped).  All loads of a round
// are issued together and re-issued until every tag matches.  Returns false on
// timeout, or when another workgroup has recorded a failure.
template <int K>
__device__ __forceinline__ bool gather_tagged(const uint64_t* const (&ptrs)[K], uint32_t tag, float (&out)[K],
                                              const uint64_t* hdr, uint32_t spin_limit) {
  bool got[K];
#pragma unroll
  for (int k = 0; k < K; ++k) got[k] = ptrs[k] == nullptr;
  for (uint32_t spin = 0;; ++spin) {
    uint64_t wv[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (!got[k]) wv[k] = get_word(ptrs[k]);
    bool all = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (!got[k]) {
        if ((uint32_t)(wv[k] >> 32) == tag) {
          out[k] = __uint_as_float((uint32_t)wv[k]);
          got[k] = true;
        } else {
          all = false;
        }
      }
    }
    if (all) return true;
    if (spin > spin_limit) return false;
    if ((spin & 1023) == 1023 && get_word(hdr + 1) != 0) return false;
  }
}

__device__ __forceinline__ void raise_failure(uint64_t* hdr) {
  __hip_atomic_store(hdr + 1, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS of one decode workgroup.
struct DecShared {
  float q[kDecodeMaxDModel];               // current layer input
  float part[kStreamers * kDecMaxC];       // per-chunk partial dot products
  float h[kDecodeMaxNeuronsPerWG];         // predictor scores of the owned neurons
  int sel[kDecodeMaxNeuronsPerWG];         // selected owned neurons, ascending
  float m[kDecodeMaxNeuronsPerWG];         // their soft-threshold values
  float c[kDecodeMaxNeuronsPerWG];         // their gated values GELU(m) * (K2^T q[r:])
  float red[kRedMax];                      // partial y, then gathered column partials
  float ycol[kDecodeMaxColsPerWG];         // owned columns of y
  float wred[8];
  float theta;
  int nsel, fail;
  uint32_t tag0;
};

// Shape of the work of one workgroup.
struct DecGeo {
  int G, w, d_model, d_ff, r, L, T;
  int n0, nown, c0, ncol;
  int CK, K2C, VC, TC, ntile, rep;
};

// Both roles execute exactly the same sequence of workgroup barriers:
//   per token:  1 (input loaded) [+2 when the input needs normalising]
//   per layer:  2 per K1 tile, then A, S, K, V, P, B, T, and either Y (last
//               layer) or C, R1, R2; the failure flag is checked after A, B, T, C.
__device__ __forceinline__ void bar() { __syncthreads(); }

// ---------------------------------------------------------------- streamer role
template <typename W>
__device__ void decode_streamer(const DecodeParams& p, const void* const* tab_k1, const DecGeo& g, DecShared& S) {
  constexpr int CN = Chunk<W>::N;
  const int sid = threadIdx.x - kWorkers, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int TILE = kStreamers * kDecMaxC;
  u32x4 pre[kDecMaxC];
  // Branch-free: chunks past the slab end re-read its last chunk (in bounds) and
  // are ignored by the dot products; with no branches the loads issue
  // back to back instead of each waiting for the previous one.
  auto load_tile = [&](int layer, int tile) {
    const char* slab = (const char*)tab_k1[layer] + (size_t)g.n0 * g.r * sizeof(W);
#pragma unroll
    for (int m = 0; m < kDecMaxC; ++m) {
      const int c = min(tile * TILE + sid + kStreamers * m, g.TC - 1);
      pre[m] = load16_stream(slab + (size_t)c * 16);
    }
  };
  load_tile(0, 0);
  for (int t = 0; t < g.T; ++t) {
    bar();
    if (p.q_prenorm) {
      bar();
      bar();
    }
    for (int l = 0; l < g.L; ++l) {
      const bool last = l == g.L - 1;
      for (int tile = 0; tile < g.ntile; ++tile) {
        if (tile > 0) load_tile(l, tile);
#pragma unroll
        for (int m = 0; m < kDecMaxC; ++m) {
          const int c = tile * TILE + sid + kStreamers * m;
          if (c < g.TC) {
            float wf[CN];
            Chunk<W>::widen(pre[m], wf);
            const float* qq = S.q + (c % g.CK) * CN;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < CN; ++e) acc += wf[e] * qq[e];
            S.part[c - tile * TILE] = acc;
          }
        }
        bar();
        // per-neuron sums of this tile's chunks (waves 4..7 take every other neuron)
        const int tb = tile * TILE, te = min(g.TC, tb + TILE);
        for (int j = tb / g.CK + wv; j <= (te - 1) / g.CK; j += 8) {
          const int a = max(j * g.CK, tb), b = min((j + 1) * g.CK, te);
          float s = 0.f;
          for (int c = a + lane; c < b; c += 64) s += S.part[c - tb];
          s = wave_sum(s);
          if (lane == 0) S.h[j] += s;
        }
        bar();
      }
      // stream the next slab while the rest of this layer runs
      const int nl = (l + 1 < g.L) ? l + 1 : ((t + 1 < g.T) ? 0 : -1);
      if (nl >= 0) load_tile(nl, 0);
      bar();  // A
      if (S.fail) return;
      bar();  // S
      bar();  // K
      bar();  // V
      bar();  // P
      bar();  // B
      if (S.fail) return;
      bar();  // T
      if (S.fail) return;
      if (last) {
        bar();  // Y
        continue;
      }
      bar();  // C
      if (S.fail) return;
      bar();  // R1
      bar();  // R2
    }
  }
}

// ---------------------------------------------------------------- worker role
template <typename W>
__device__ void decode_worker(const DecodeParams& p, const void* const* tab_k2, const void* const* tab_v,
                              const DecGeo& g, DecShared& S) {
  constexpr int CN = Chunk<W>::N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int TILE = kStreamers * kDecMaxC;
  const int d_model = g.d_model, G = g.G, w = g.w;
  uint32_t tag = S.tag0;

  for (int t = 0; t < g.T; ++t) {
    for (int c = tid; c < d_model; c += kWorkers) S.q[c] = p.q_in[(size_t)t * d_model + c];
    bar();
    if (p.q_prenorm) {
      float ss = 0.f;
      for (int c = tid; c < d_model; c += kWorkers) ss += S.q[c] * S.q[c];
      ss = wave_sum(ss);
      if (lane == 0) S.wred[wv] = ss;
      bar();
      const float inv = 1.f / sqrtf((S.wred[0] + S.wred[1] + S.wred[2] + S.wred[3]) / (float)d_model + p.eps);
      for (int c = tid; c < d_model; c += kWorkers) S.q[c] *= inv;
      bar();
    }
    for (int l = 0; l < g.L; ++l) {
      const bool last = l == g.L - 1;
      const uint32_t tagA = ++tag, tagB = ++tag, tagC = last ? 0u : ++tag;
      const size_t trow = (size_t)t * p.total_layers + p.layer_offset + l;
      if (p.tr_q && w == 0)
        for (int c = tid; c < d_model; c += kWorkers) p.tr_q[trow * d_model + c] = S.q[c];
      for (int j = tid; j < g.nown; j += kWorkers) S.h[j] = 0.f;

      // ---------------- predictor: the streamers form chunk dots, all waves sum them
      for (int tile = 0; tile < g.ntile; ++tile) {
        bar();
        const int tb = tile * TILE, te = min(g.TC, tb + TILE);
        for (int j = tb / g.CK + wv; j <= (te - 1) / g.CK; j += 8) {
          const int a = max(j * g.CK, tb), b = min((j + 1) * g.CK, te);
          float s = 0.f;
          for (int c = a + lane; c < b; c += 64) s += S.part[c - tb];
          s = wave_sum(s);
          if (lane == 0) S.h[j] += s;
        }
        bar();
      }

      // ---------------- exchange A: moments of the predictor scores -> theta
      if (wv == 0) {
        float s = 0.f;
        for (int j = lane; j < g.nown; j += 64) s += S.h[j];
        const float mean_w = wave_sum(s) / (float)g.nown;
        float q2 = 0.f;
        for (int j = lane; j < g.nown; j += 64) {
          const float dv = S.h[j] - mean_w;
          q2 += dv * dv;
        }
        const float m2_w = wave_sum(q2);
        if (lane < kRep) {
          uint64_t* dst = p.stats + (size_t)lane * p.stats_stride + 2 * w;
          put_tagged(dst, mean_w, tagA);
          put_tagged(dst + 1, m2_w, tagA);
        }
        const uint64_t* src = p.stats + (size_t)g.rep * p.stats_stride;
        constexpr int KA = 8;  // 4 records (G <= 256) x 2 words per lane
        const uint64_t* ptrs[KA];
#pragma unroll
        for (int k = 0; k < KA / 2; ++k) {
          const int gg = lane + 64 * k;
          ptrs[2 * k] = gg < G ? src + 2 * gg : nullptr;
          ptrs[2 * k + 1] = gg < G ? src + 2 * gg + 1 : nullptr;
        }
        float vals[KA];
        const bool ok = gather_tagged<KA>(ptrs, tagA, vals, p.hdr, p.spin_limit);
        Moments acc{0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KA / 2; ++k) {
          const int gg = lane + 64 * k;
          if (gg < G) {
            const float ng = (float)((int)((int64_t)(gg + 1) * g.d_ff / G) - (int)((int64_t)gg * g.d_ff / G));
            acc = merge(acc, Moments{ng, vals[2 * k], vals[2 * k + 1]});
          }
        }
        const Moments tot = wave_merge(acc);
        if (lane == 0) S.theta = tot.mean + sqrtf(tot.m2 / (float)g.d_ff) * p.z;
        if (__builtin_amdgcn_ballot_w64(!ok) != 0 && lane == 0) {
          S.fail = 1;
          raise_failure(p.hdr);
        }
      }
      bar();  // A
      if (S.fail) return;
      const float theta = S.theta;

      // ---------------- selection of the owned neurons (ascending)
      if (wv == 0) {
        int base = 0;
        for (int j0 = 0; j0 < g.nown; j0 += 64) {
          const int j = j0 + lane;
          const bool on = j < g.nown && S.h[j] > theta;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
          const int pos =
              base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
          if (on) {
            S.sel[pos] = j;
            S.m[pos] = S.h[j] - theta;
          }
          base += __builtin_popcountll(bal);
        }
        if (lane == 0) S.nsel = base;
      }
      bar();  // S
      const int nsel = S.nsel;

      // ---------------- K2 gather-dot and gate: c = GELU(m) * (K2^T q[r:])
      for (int e = wv; e < nsel; e += kWorkers / 64) {
        const char* row = (const char*)tab_k2[l] + (size_t)(g.n0 + S.sel[e]) * (d_model - g.r) * sizeof(W);
        float s = 0.f;
        for (int cc = lane; cc < g.K2C; cc += 64) {
          float wf[CN];
          Chunk<W>::widen(load16(row + (size_t)cc * 16), wf);
          const float* qq = S.q + g.r + cc * CN;
#pragma unroll
          for (int e2 = 0; e2 < CN; ++e2) s += wf[e2] * qq[e2];
        }
        s = wave_sum(s);
        if (lane == 0) S.c[e] = gelu_tanh(S.m[e]) * s;
      }
      bar();  // K

      // ---------------- V rows: partial y of this workgroup, staged in LDS
      for (int vc = tid; vc < g.VC; vc += kWorkers) {
        float acc[CN];
#pragma unroll
        for (int e2 = 0; e2 < CN; ++e2) acc[e2] = 0.f;
        for (int e0 = 0; e0 < nsel; e0 += 4) {
          u32x4 raw[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (e0 + u < nsel)
              raw[u] = load16((const char*)tab_v[l] + (size_t)(g.n0 + S.sel[e0 + u]) * d_model * sizeof(W) +
                              (size_t)vc * 16);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (e0 + u < nsel) {
              float wf[CN];
              Chunk<W>::widen(raw[u], wf);
              const float cf = S.c[e0 + u];
#pragma unroll
              for (int e2 = 0; e2 < CN; ++e2) acc[e2] += cf * wf[e2];
            }
          }
        }
#pragma unroll
        for (int e2 = 0; e2 < CN; ++e2) S.red[vc * CN + e2] = acc[e2];
      }
      bar();  // V

      // ---------------- exchange B: publish partial y (and the selected count)
      {
        uint64_t* mine = p.part + (size_t)w * p.part_stride;
        for (int c = tid; c < d_model; c += kWorkers) put_tagged(mine + c, S.red[c], tagB);
        if (tid == 0) put_tagged_u32(mine + d_model, (uint32_t)nsel, tagB);
      }
      bar();  // P
      // gather the owned columns of every workgroup's partial
      {
        bool okB = true;
        const int total = G * g.ncol;
        constexpr int KB = 8;
        for (int i0 = 0; i0 < total; i0 += kWorkers * KB) {
          const uint64_t* ptrs[KB];
#pragma unroll
          for (int k = 0; k < KB; ++k) {
            const int i = i0 + tid + kWorkers * k;
            const int gg = i / g.ncol, cc = i - gg * g.ncol;
            ptrs[k] = i < total ? p.part + (size_t)gg * p.part_stride + g.c0 + cc : nullptr;
          }
          float vals[KB];
          okB &= gather_tagged<KB>(ptrs, tagB, vals, p.hdr, p.spin_limit);
#pragma unroll
          for (int k = 0; k < KB; ++k) {
            const int i = i0 + tid + kWorkers * k;
            if (i < total) S.red[i] = vals[k];
          }
        }
        if (!okB) S.fail = 1;
      }
      bar();  // B
      if (S.fail) {
        if (tid == 0) raise_failure(p.hdr);
        return;
      }
      // fixed-order sum over the G partials of each owned column
      for (int cc = wv; cc < g.ncol; cc += kWorkers / 64) {
        float s = 0.f;
        for (int gg = lane; gg < G; gg += 64) s += S.red[gg * g.ncol + cc];
        s = wave_sum(s);
        if (lane == 0) S.ycol[cc] = s;
      }
      // trace: threshold, counts and indices of this layer
      if ((p.tr_counts || p.tr_idx || p.tr_theta) && wv == 0) {
        bool okT = true;
        int before = 0, all = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
          const int gg = g0 + lane;
          const uint64_t* ptr[1] = {gg < G ? p.part + (size_t)gg * p.part_stride + d_model : nullptr};
          float v1[1] = {0.f};
          okT &= gather_tagged<1>(ptr, tagB, v1, p.hdr, p.spin_limit);
          const int cnt = gg < G ? (int)__float_as_uint(v1[0]) : 0;
          before += wave_sum_int(gg < w ? cnt : 0);
          all += wave_sum_int(cnt);
        }
        if (p.tr_idx)
          for (int e = lane; e < nsel; e += 64) {
            const int64_t pos = before + e;
            if (pos < p.tr_cap) p.tr_idx[trow * p.tr_cap + pos] = g.n0 + S.sel[e];
          }
        if (w == 0 && lane == 0) {
          if (p.tr_counts) p.tr_counts[trow] = all;
          if (p.tr_theta) p.tr_theta[trow] = theta;
        }
        if (__builtin_amdgcn_ballot_w64(!okT) != 0 && lane == 0) S.fail = 1;
      }
      bar();  // T
      if (S.fail) {
        if (tid == 0) raise_failure(p.hdr);
        return;
      }
      if (last) {
        for (int cc = tid; cc < g.ncol; cc += kWorkers) p.y_out[(size_t)t * d_model + g.c0 + cc] = S.ycol[cc];
        bar();  // Y
        continue;
      }

      // ---------------- exchange C: owned columns of y -> every workgroup
      {
        for (int i = tid; i < kRep * g.ncol; i += kWorkers) {
          const int rp = i / g.ncol, cc = i - rp * g.ncol;
          put_tagged(p.ycol + (size_t)rp * p.ycol_stride + g.c0 + cc, S.ycol[cc], tagC);
        }
        bool okC = true;
        const uint64_t* src = p.ycol + (size_t)g.rep * p.ycol_stride;
        constexpr int KC = 8;
        for (int c00 = 0; c00 < d_model; c00 += kWorkers * KC) {
          const uint64_t* ptrs[KC];
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const int c = c00 + tid + kWorkers * k;
            ptrs[k] = c < d_model ? src + c : nullptr;
          }
          float vals[KC];
          okC &= gather_tagged<KC>(ptrs, tagC, vals, p.hdr, p.spin_limit);
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const int c = c00 + tid + kWorkers * k;
            if (c < d_model) S.q[c] = vals[k];
          }
        }
        if (!okC) S.fail = 1;
      }
      bar();  // C
      if (S.fail) {
        if (tid == 0) raise_failure(p.hdr);
        return;
      }
      // RMS normalisation (identical order in every workgroup)
      {
        float ss = 0.f;
        for (int c = tid; c < d_model; c += kWorkers) ss += S.q[c] * S.q[c];
        ss = wave_sum(ss);
        if (lane == 0) S.wred[wv] = ss;
      }
      bar();  // R1
      {
        const float inv = 1.f / sqrtf((S.wred[0] + S.wred[1] + S.wred[2] + S.wred[3]) / (float)d_model + p.eps);
        for (int c = tid; c < d_model; c += kWorkers) S.q[c] *= inv;
      }
      bar();  // R2
    }
  }
  if (w == 0 && tid == 0) __hip_atomic_store(p.hdr, (uint64_t)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename W>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeParams p) {
  constexpr int CN = Chunk<W>::N;
  __shared__ DecShared S;
  // the layer tables are read in place from the kernel-argument segment
  // (scalar loads), never copied into registers
  const DecodeParams* kp = (const DecodeParams*)__builtin_amdgcn_kernarg_segment_ptr();
  DecGeo g;
  g.G = gridDim.x;
  g.w = blockIdx.x;
  g.d_model = p.d_model;
  g.d_ff = p.d_ff;
  g.r = p.r;
  g.L = p.n_layers;
  g.T = p.T;
  g.n0 = (int)((int64_t)g.w * g.d_ff / g.G);
  g.nown = (int)((int64_t)(g.w + 1) * g.d_ff / g.G) - g.n0;
  g.c0 = (int)((int64_t)g.w * g.d_model / g.G);
  g.ncol = (int)((int64_t)(g.w + 1) * g.d_model / g.G) - g.c0;
  g.CK = g.r / CN;
  g.K2C = (g.d_model - g.r) / CN;
  g.VC = g.d_model / CN;
  g.TC = g.nown * g.CK;
  g.ntile = (g.TC + kStreamers * kDecMaxC - 1) / (kStreamers * kDecMaxC);
  g.rep = xcc_id();
  if (threadIdx.x == 0) {
    S.tag0 = (uint32_t)get_word(p.hdr);
    S.fail = 0;
  }
  __syncthreads();
  if (threadIdx.x < kWorkers)
    decode_worker<W>(p, kp->k2t, kp->v, g, S);
  else
    decode_streamer<W>(p, kp->k1t, g, S);
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct DecodeLayout {
  size_t hdr, stats, part, ycol, qbuf, total;
  int stats_stride, part_stride, ycol_stride;
};

static DecodeLayout decode_layout(int64_t d_model, int64_t T, int grid, int n_layers) {
  DecodeLayout L;
  L.stats_stride = (int)round_up((size_t)2 * grid + 64, 512);      // words; replicas 4 KB+ apart
  L.part_stride = (int)round_up((size_t)d_model + 1, 16);           // words, 128-byte rows
  L.ycol_stride = (int)round_up((size_t)d_model + 64, 512);
  size_t off = 0;
  L.hdr = off;
  off += 256;
  L.stats = off;
  off += round_up((size_t)kRep * L.stats_stride * 8, 256);
  L.part = off;
  off += round_up((size_t)grid * L.part_stride * 8, 256);
  L.ycol = off;
  off += round_up((size_t)kRep * L.ycol_stride * 8, 256);
  L.qbuf = off;
  if (n_layers > kDecodeMaxLayersPerLaunch) off += 2 * round_up((size_t)T * d_model * 4, 256);
  L.total = off;
  return L;
}

int decode_grid(int64_t d_ff) {
  const int cus = device_cu_count();
  return (int)(d_ff < cus ? d_ff : cus);
}

size_t decode_workspace_bytes(int64_t d_model, int64_t d_ff, int n_layers, int64_t T, int grid) {
  (void)d_ff;
  return decode_layout(d_model, T, grid, n_layers).total;
}

template <typename W>
static hipError_t launch_decode_t(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                  const float* q, int64_t T, float* y, float eps, double z,
                                  const spark_ffn_trace* trace, void* ws, hipStream_t st) {
  const int grid = decode_grid(s.d_ff);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<W>, kDecodeThreads, 0);
  if (e != hipSuccess) return e;
  if ((int64_t)per_cu * device_cu_count() < grid) return hipErrorCooperativeLaunchTooLarge;
  const DecodeLayout Lo = decode_layout(s.d_model, T, grid, n_layers);
  char* base = (char*)ws;
  float* qbuf[2] = {(float*)(base + Lo.qbuf), (float*)(base + Lo.qbuf + round_up((size_t)T * s.d_model * 4, 256))};
  for (int lo = 0, seg = 0; lo < n_layers; lo += kDecodeMaxLayersPerLaunch, ++seg) {
    const int nl = n_layers - lo < kDecodeMaxLayersPerLaunch ? n_layers - lo : kDecodeMaxLayersPerLaunch;
    DecodeParams p;
    for (int i = 0; i < kDecodeMaxLayersPerLaunch; ++i) {
      const spark_ffn_weights& lw = layers[lo + (i < nl ? i : 0)];
      p.k1t[i] = lw.k1t;
      p.k2t[i] = lw.k2t;
      p.v[i] = lw.v;
    }
    p.n_layers = nl;
    p.layer_offset = lo;
    p.total_layers = n_layers;
    p.d_model = (int)s.d_model;
    p.d_ff = (int)s.d_ff;
    p.r = (int)s.r;
    p.T = (int)T;
    p.z = (float)z;
    p.eps = eps;
    const bool first = lo == 0, lastseg = lo + nl >= n_layers;
    p.q_in = first ? q : qbuf[(seg - 1) & 1];
    p.q_prenorm = first ? 0 : 1;
    p.y_out = lastseg ? y : qbuf[seg & 1];
    p.tr_counts = trace ? trace->counts : nullptr;
    p.tr_idx = trace ? trace->idx : nullptr;
    p.tr_theta = trace ? trace->theta : nullptr;
    p.tr_q = trace ? trace->q_in : nullptr;
    p.tr_cap = trace ? trace->cap : 0;
    p.hdr = (uint64_t*)(base + Lo.hdr);
    p.stats = (uint64_t*)(base + Lo.stats);
    p.part = (uint64_t*)(base + Lo.part);
    p.ycol = (uint64_t*)(base + Lo.ycol);
    p.stats_stride = Lo.stats_stride;
    p.part_stride = Lo.part_stride;
    p.ycol_stride = Lo.ycol_stride;
    p.spin_limit = 1u << 22;
    void* args[] = {&p};
    e = hipLaunchCooperativeKernel((const void*)decode_kernel<W>, dim3(grid), dim3(kDecodeThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_decode(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers, const float* q,
                         int64_t T, float* y, float eps, double z, const spark_ffn_trace* trace, void* ws,
                         hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (s.wdtype == SPARK_BF16) return launch_decode_t<bf16_t>(s, layers, n_layers, q, T, y, eps, z, trace, ws, st);
  return launch_decode_t<float>(s, layers, n_layers, q, T, y, eps, z, trace, ws, st);
}

}  // namespace spark
