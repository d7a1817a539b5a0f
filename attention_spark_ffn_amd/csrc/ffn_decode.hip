// Spark FFN decode: a persistent kernel that runs the whole stack of
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
// predictor scores -> theta; B: per-workgroup selected list, a 64-bit mask
// and the gated values -> every workgroup; C: owned columns of y -> every
// workgroup) move 64-bit words that carry the value and a 32-bit tag.
// Writers store them with device-scope relaxed atomics (coherent across the
// eight XCD L2 caches); readers poll until the tag of the exchange appears,
// so no cross-XCD fence is needed.  Every record is written to several
// copies, each read by a fixed share of the workgroups (16 copies of the
// statistics, 2 of the selection records, one per XCD of the layer output:
// measured).  In exchange B only the two mask words are
// polled: the entries are stored before them and read once the mask is seen
// (an entry still without its tag is polled), which keeps the polling
// traffic of 256 readers to two words per record.
// Every wait is bounded: on timeout the kernel records a failure in the
// workspace header (the failed call's mark and a count of failed calls), the
// workgroups write NaN over the output columns they own and leave, and
// workgroup 0 still advances the tag in the header past every tag the call
// owns, so no word of the failed call can satisfy a wait of a later one.
#include <mutex>

#include "common.hpp"
#include "exchange.hpp"
#include "internal.hpp"

namespace spark {

constexpr int kDecMaxC = 21;   // K1 chunks (16 B) held per streamer thread (a 36 x 1152 bf16 slab)
constexpr int kStreamers = 256;
constexpr int kWorkers = 256;
// Copies of the broadcast records of each exchange; workgroup w reads copy
// (x + 8 ((w / 8) % 2)) % kRep* with x its XCD (measured: statistics 16
// copies, 16 readers each; selection records 2, written fastest; the layer
// output one per XCD)
constexpr int kRepA = 16;      // statistics
constexpr int kRepB = 2;       // selection records
constexpr int kRepC = 8;       // layer output
constexpr int kCand = 10;      // owned neurons whose K2 dot is formed before theta is known
constexpr int kRecWords = 16;  // selected-list record: 2 mask words + 14 entries
constexpr int kRecEntries = kRecWords - 2;
constexpr int kRecRow = 256;   // records are word-major: word k of workgroup w at k * kRecRow + w
constexpr int kSpecE = 10;     // entries polled together with the mask words
constexpr int kK2Step = 9;     // K2 chunks per lane in flight in a candidate dot
constexpr int kQPer = 9;       // q chunks a streamer keeps in registers (period of its q offsets)
constexpr int kOvfWords = kDecodeMaxNeuronsPerWG - kRecEntries;

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
  uint64_t* hdr;    // [0]: tag before the next call, [1]: mark (tag0 + 1) of the last failed call, [2]: failed
                    // calls, [3]: bound of every wait when nonzero (test hook)
  uint64_t* stats;  // kRepA x stats_stride: means of all workgroups, then their M2 (kRecRow apart)
  uint64_t* rec;    // kRepB x rec_stride: selected-list record per workgroup
  uint64_t* ovf;    // G x kOvfWords: list entries past the record
  uint64_t* ycol;   // kRepC x ycol_stride: owned columns of y
  int stats_stride, rec_stride, ycol_stride;
  uint32_t spin_limit;
};

// LDS of one decode workgroup.
struct DecShared {
  alignas(16) float q[kDecodeMaxDModel];  // current layer input
  union {
    float part[kStreamers * kDecMaxC + 64];  // per-chunk partial dot products (+ a dummy slot)
  } u;
  float h[kDecodeMaxNeuronsPerWG];   // predictor scores of the owned neurons
  float g[kDecodeMaxNeuronsPerWG];   // K2^T q[r:] of the owned neurons (candidates, then misses)
  int cnt[256];                      // selected count of every workgroup
  int off[256];                      // exclusive prefix of cnt
  float colpart[4][16];              // per-wave sums of the owned columns
  float wred[8];
  float theta;
  int ntot, fail;
  uint32_t tag0;
  uint32_t spin_limit;  // polling rounds a wait may take
  uint32_t poison;      // XORed into the tag exchange A waits for (nonzero: the test hook's forced failure)
  uint32_t aflag;       // layer key (token * layers + layer + 1) whose theta is in S.theta
  uint32_t dotcnt;      // candidate K2 dot waves done (3 per layer)
  uint64_t fmark;       // tag0 + 1: the failure mark of this call
};

// Shape of the work of one workgroup.
struct DecGeo {
  int G, w, d_model, d_ff, r, L, T;
  int n0, nown, c0, ncol, ch0, nch;
  int CK, K2C, TC, ntile, rep;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }

// First neuron of workgroup g (g * d_ff < 2^32 under the decode limits).
__device__ __forceinline__ int own_first(int g, int d_ff, int G) {
  return (int)((uint32_t)g * (uint32_t)d_ff / (uint32_t)G);
}

// Output columns owned by workgroup wg: the workgroups of one XCD
// (wg = x + 8j) own one contiguous range, so each V row segment is read once
// per XCD.  Ranges are whole 16-byte chunks of a V row (cn elements each).
__device__ __forceinline__ void col_range(int wg, int G, int d_model, int cn, int& c0, int& ncol) {
  const int o = (G % 8 == 0) ? (wg & 7) * (G / 8) + (wg >> 3) : wg;
  const int vch = d_model / cn;  // 16-byte chunks per V row
  const int ch0 = (int)((int64_t)o * vch / G);
  c0 = ch0 * cn;
  ncol = ((int)((int64_t)(o + 1) * vch / G) - ch0) * cn;
}

// Both roles execute exactly the same sequence of workgroup barriers:
//   per token:  1 (input loaded) [+2 when the input needs normalising]
//   per layer:  2 per K1 tile, then [T1, T2: workgroup 0, when a trace is
//               asked for], V, and either Y (last layer) or C; the failure
//               flag is read after V and C.
// Inside a layer the waves also signal each other through LDS flags (theta
// known, candidate K2 dots done), which the waves that wait on them poll
// with a bound.
__device__ __forceinline__ void bar() { __syncthreads(); }

// Wait (bounded) until the LDS word *w reaches v; false on timeout.
__device__ __forceinline__ bool lds_wait_ge(const uint32_t* w, uint32_t v) {
  bool ok = true;
  for (uint32_t sp = 0; __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < v; ++sp) {
    if (sp > (1u << 22)) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return ok;
}
// Publish v in the LDS word *w after this wave's earlier LDS writes.
__device__ __forceinline__ void lds_signal(uint32_t* w, uint32_t v) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}



// Per-neuron sums of one tile's chunk products.  Wave wv takes neurons
// wv, wv + 8, ...; in the common case (one tile, rows of at most 192 chunks,
// at most 64 neurons) all of a wave's LDS reads are issued before any sum.
__device__ __forceinline__ void reduce_tile(const DecGeo& g, DecShared& S, int tile, int lane, int wv, float qs) {
  const int TILE = kStreamers * kDecMaxC;
  const int tb = tile * TILE, te = min(g.TC, tb + TILE);
  if (g.ntile == 1 && g.CK <= 192) {
    float v[8][3];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = wv + 8 * u;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int c = j * g.CK + lane + 64 * k;
        const bool ok = j < g.nown && lane + 64 * k < g.CK;
        v[u][k] = S.u.part[ok ? c : TILE];
        v[u][k] = ok ? v[u][k] : 0.f;
      }
    }
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = (v[u][0] + v[u][1]) + v[u][2];
    int u;
    const float s = wave_colsum<8>(t, lane, u);
    const int j = wv + 8 * u;
    if ((lane & 7) == 0 && j < g.nown) S.h[j] = s * qs;
    return;
  }
  for (int j = tb / g.CK + wv; j <= (te - 1) / g.CK; j += 8) {
    const int a = max(j * g.CK, tb), b = min((j + 1) * g.CK, te);
    float s = 0.f;
    for (int c = a + lane; c < b; c += 64) s += S.u.part[c - tb];
    s = wave_sum_dpp(s);
    if (lane == 0) S.h[j] += s * qs;
  }
}

// ---------------------------------------------------------------- streamer role
template <typename W>
__device__ void decode_streamer(const DecodeParams& p, const void* const* tab_k1, const void* const* tab_v, const DecGeo& g, DecShared& S) {
  constexpr int CN = Chunk<W>::N;
  const int sid = threadIdx.x - kWorkers, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int TILE = kStreamers * kDecMaxC;
  u32x4 pre[kDecMaxC];
  // q offsets of the first kQPer register chunks of tile 0
  int qoff[kQPer];
#pragma unroll
  for (int m = 0; m < kQPer; ++m) {
    const int c = sid + kStreamers * m;
    qoff[m] = c < g.TC ? (c % g.CK) * CN : 0;
  }
  // Branch-free: chunks past the slab end re-read its last chunk (in bounds) and
  // their products go to a dummy slot; with no branches the loads issue back to
  // back and the LDS reads of consecutive chunks overlap.
  // The chunk offsets are formed anew at every call (from an opaque copy of
  // the thread index) rather than held in registers for the whole kernel.
  // Register chunks [m0, m1) of a tile.
  auto load_part = [&](int layer, int tile, int m0, int m1) {
    const char* slab = (const char*)tab_k1[layer] + (size_t)g.n0 * g.r * sizeof(W);
    int s0 = tile * TILE + sid;
    asm volatile("" : "+v"(s0));
#pragma unroll
    for (int m = 0; m < kDecMaxC; ++m) {
      if (m < m0 || m >= m1) continue;
      const int c = min(s0 + kStreamers * m, g.TC - 1);
      pre[m] = load16_stream(slab + (uint32_t)c * 16u);
    }
  };
  auto load_tile = [&](int layer, int tile) { load_part(layer, tile, 0, kDecMaxC); };
  // The next slab is streamed from the moment theta is known: its loads then
  // overlap the list exchange and the V product.  (Issued earlier they would
  // queue in front of the statistics exchange and the candidate K2 loads;
  // issued later, in front of the exchange of the layer output, or too late
  // to land before the next predictor product.)
  auto prefetch_part = [&](int t, int l, int m0, int m1) {
    const int nl = (l + 1 < g.L) ? l + 1 : ((t + 1 < g.T) ? 0 : -1);
    if (nl >= 0) load_part(nl, 0, m0, m1);
  };
  // chunk c of the slab multiplies q[(c % CK) * CN ...]; with c = sid + 256 m
  // that offset has period kQPer in m when 256 kQPer is a multiple of CK
  const bool qreg = g.ntile == 1 && (kStreamers * kQPer) % g.CK == 0;
  const bool trace_here = g.w == 0 && (p.tr_idx || p.tr_counts || p.tr_theta);
  load_tile(0, 0);
  uint32_t vsink = 0;  // the V touches' loaded words (never used)
  float qs = 1.f;  // scale of the q held in LDS (its RMS normalisation, applied to the products)
  for (int t = 0; t < g.T; ++t) {
    qs = 1.f;
    bar();
    if (p.q_prenorm) {
      bar();
      bar();
    }
    for (int l = 0; l < g.L; ++l) {
      const bool last = l == g.L - 1;
      if (qreg) {
        // one tile, and the q offsets of a thread's chunks repeat every kQPer
        // chunks: the kQPer distinct q chunks are read from LDS once
        float qv[kQPer][CN];
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
          const f32x4* qq = reinterpret_cast<const f32x4*>(S.q + qoff[i]);
#pragma unroll
          for (int e4 = 0; e4 < CN / 4; ++e4) {
            const f32x4 x = qq[e4];
            qv[i][4 * e4] = x.x;
            qv[i][4 * e4 + 1] = x.y;
            qv[i][4 * e4 + 2] = x.z;
            qv[i][4 * e4 + 3] = x.w;
          }
        }
#pragma unroll
        for (int m = 0; m < kDecMaxC; ++m) {
          const int c = sid + kStreamers * m;
          float wf[CN];
          Chunk<W>::widen(pre[m], wf);
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < CN; ++e) acc += wf[e] * qv[m % kQPer][e];
          S.u.part[c < g.TC ? c : TILE] = acc;
          if (m % 3 == 2) __builtin_amdgcn_sched_barrier(0);  // keep few chunks' conversions live
        }
        asm volatile("" :: "v"(vsink));  // keeps the V touches (complete long before this point)
        bar();
        reduce_tile(g, S, 0, lane, wv, qs);
        bar();
      }
      for (int tile = 0; !qreg && tile < g.ntile; ++tile) {
        if (tile > 0) load_tile(l, tile);
#pragma unroll
        for (int m = 0; m < kDecMaxC; ++m) {
          const int c = tile * TILE + sid + kStreamers * m;
          const bool ok = c < g.TC;
          const int qo = ok ? (c % g.CK) * CN : 0;
          float wf[CN];
          Chunk<W>::widen(pre[m], wf);
          const f32x4* qq = reinterpret_cast<const f32x4*>(S.q + qo);  // 16-byte aligned
          float acc = 0.f;
#pragma unroll
          for (int e4 = 0; e4 < CN / 4; ++e4) {
            const f32x4 qv = qq[e4];
            acc += wf[4 * e4] * qv.x + wf[4 * e4 + 1] * qv.y + wf[4 * e4 + 2] * qv.z + wf[4 * e4 + 3] * qv.w;
          }
          S.u.part[ok ? c - tile * TILE : TILE] = acc;
          // at most three chunks' q reads in flight: enough to cover the LDS
          // latency without holding every chunk's q in registers
          if (m % 3 == 2) __builtin_amdgcn_sched_barrier(0);
        }
        bar();
        // per-neuron sums of this tile's chunks (waves 4..7 take every other neuron)
        reduce_tile(g, S, tile, lane, wv, qs);
        bar();
      }
      // the next slab streams from the moment theta is known
      lds_wait_ge(&S.aflag, (uint32_t)(t * g.L + l + 1));
      prefetch_part(t, l, 0, kDecMaxC);
      // ... and the V rows of this workgroup's selected neurons are touched
      // (one 4-byte load per 128-byte line), so that the column owners of
      // every XCD find them in the caches when the selection lists arrive
      {
        const float th = S.theta;
        const bool on = lane < g.nown && S.h[lane < 64 ? lane : 0] > th;
        uint64_t M = __builtin_amdgcn_ballot_w64(on);
        const int sw = wv - 4;
        for (int k = 0; M; ++k) {
          const int j = __builtin_ctzll(M);
          M &= M - 1;
          if ((k & 3) != sw) continue;
          const char* row = (const char*)tab_v[l] + (size_t)(g.n0 + j) * (size_t)g.d_model * sizeof(W);
          const int lines = (g.d_model * (int)sizeof(W) + 127) / 128;
          for (int c = lane; c < lines; c += 64) vsink ^= *reinterpret_cast<const uint32_t*>(row + (size_t)c * 128);
        }
      }
      if (trace_here) {
        bar();  // T1
        bar();  // T2
      }
      bar();  // V
      if (S.fail) return;
      if (last) {
        bar();  // Y
        continue;
      }
      bar();  // C
      if (S.fail) return;
      qs = 1.f / sqrtf((S.wred[0] + S.wred[1] + S.wred[2] + S.wred[3]) / (float)g.d_model + p.eps);
    }
  }
}

// K2^T q[r:] for one owned neuron by a row of 16 lanes (the four rows of a
// wave take four neurons).  Lane s of the row takes chunks s, s + 16, ...;
// all kK2Step loads of a step are issued before any is used, so a row of up
// to 16 kK2Step chunks costs one memory round trip.
template <typename W>
__device__ __forceinline__ float k2_dot_row16(const char* row, const float* qr, int K2C, int s) {
  constexpr int CN = Chunk<W>::N;
  float acc = 0.f;
  for (int c0 = 0; c0 < K2C; c0 += 16 * kK2Step) {
    u32x4 raw[kK2Step];
#pragma unroll
    for (int i = 0; i < kK2Step; ++i) raw[i] = load16(row + (size_t)min(c0 + s + 16 * i, K2C - 1) * 16);
#pragma unroll
    for (int i = 0; i < kK2Step; ++i) {
      const int cc = c0 + s + 16 * i;
      float wf[CN];
      Chunk<W>::widen(raw[i], wf);
      const f32x4* qq = reinterpret_cast<const f32x4*>(qr + (cc < K2C ? cc : 0) * CN);  // 16-byte aligned
      float a = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < CN / 4; ++e4) {
        const f32x4 qv = qq[e4];
        a += wf[4 * e4] * qv.x + wf[4 * e4 + 1] * qv.y + wf[4 * e4 + 2] * qv.z + wf[4 * e4 + 3] * qv.w;
      }
      acc += cc < K2C ? a : 0.f;
    }
  }
  return row16_sum(acc);
}

// This thread's share of the V product: the selected neurons of one record
// (workgroup gg's, whose selection mask Mg is known), NCH owned 16-byte
// chunks of each V row.  The loads of the first kSpecE entries' gated values
// and of their V chunks are all issued before any is used (one memory round
// trip); every entry word carries the exchange tag, and one that is not yet
// visible is polled again.  Later entries (a record with more selected
// neurons) are read one at a time.  Returns false if an entry never appeared.
template <typename W, int NCH>
__device__ __forceinline__ bool v_record(const DecodeParams& p, const DecShared& S, const char* vbase, size_t vrow,
                                         uint64_t Mg, int nb, const uint64_t* rp, int gg, uint32_t tagB,
                                         float (&acc)[2 * Chunk<W>::N]) {
  constexpr int CN = Chunk<W>::N;
  const int n = __builtin_popcountll(Mg);
  uint64_t mm = Mg;
  int jv[kSpecE];
#pragma unroll
  for (int e = 0; e < kSpecE; ++e) {
    jv[e] = mm ? __builtin_ctzll(mm) : 0;
    mm &= mm - 1;
  }
  uint64_t ew[kSpecE];
#pragma unroll
  for (int e = 0; e < kSpecE; ++e) ew[e] = e < n ? get_word(rp + (size_t)(2 + e) * kRecRow) : 0;
  u32x4 raw[kSpecE][NCH];
#pragma unroll
  for (int e = 0; e < kSpecE; ++e)
    if (e < n)
#pragma unroll
      for (int hh = 0; hh < NCH; ++hh) raw[e][hh] = load16(vbase + (size_t)(nb + jv[e]) * vrow + hh * 16);
  bool ok = true;
  float cv[kSpecE];
#pragma unroll
  for (int e = 0; e < kSpecE; ++e) {
    cv[e] = __uint_as_float((uint32_t)ew[e]);
    if (e < n && (uint32_t)(ew[e] >> 32) != tagB) {  // not yet visible: poll it
      const uint64_t* ep[1] = {rp + (size_t)(2 + e) * kRecRow};
      float v1[1];
      ok = ok && gather_tagged<1>(ep, tagB, v1, p.hdr, S.fmark, S.spin_limit);
      cv[e] = ok ? v1[0] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < kSpecE; ++e)
    if (e < n)
#pragma unroll
      for (int hh = 0; hh < NCH; ++hh) {
        float wf[CN];
        Chunk<W>::widen(raw[e][hh], wf);
#pragma unroll
        for (int i = 0; i < CN; ++i) acc[hh * CN + i] += cv[e] * wf[i];
      }
  for (int e = kSpecE; e < n && ok; ++e) {
    const int j = __builtin_ctzll(mm);
    mm &= mm - 1;
    const uint64_t* ep[1] = {e < kRecEntries ? rp + (size_t)(2 + e) * kRecRow
                                             : p.ovf + (size_t)gg * kOvfWords + (e - kRecEntries)};
    float v1[1];
    ok = gather_tagged<1>(ep, tagB, v1, p.hdr, S.fmark, S.spin_limit);
#pragma unroll
    for (int hh = 0; hh < NCH; ++hh) {
      float wf[CN];
      Chunk<W>::widen(load16(vbase + (size_t)(nb + j) * vrow + hh * 16), wf);
#pragma unroll
      for (int i = 0; i < CN; ++i) acc[hh * CN + i] += v1[0] * wf[i];
    }
  }
  return ok;
}

// ---------------------------------------------------------------- worker role
template <typename W>
__device__ void decode_worker(const DecodeParams& p, const void* const* tab_k2, const void* const* tab_v,
                              const DecGeo& g, DecShared& S) {
  constexpr int CN = Chunk<W>::N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int TILE = kStreamers * kDecMaxC;
  const int d_model = g.d_model, G = g.G, w = g.w;
  const size_t k2row = (size_t)(d_model - g.r) * sizeof(W);
  const size_t vrow = (size_t)d_model * sizeof(W);
  uint32_t tag = S.tag0;
  // neurons owned by the workgroups whose statistics this lane combines, and
  // the first neuron of the workgroup whose record this thread places
  float ngk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int gg = lane + 64 * k;
    ngk[k] = gg < G ? (float)(own_first(gg + 1, g.d_ff, G) - own_first(gg, g.d_ff, G)) : 0.f;
  }
  const int nb_rec = own_first(tid < G ? tid : 0, g.d_ff, G);
  const bool trace_here = w == 0 && (p.tr_idx || p.tr_counts || p.tr_theta);
  // a failed call: mark it, and NaN over the owned output columns of every token
  auto fail_out = [&]() {
    if (tid == 0) raise_failure(p.hdr, S.fmark);
    if (tid < g.ncol)
      for (int t2 = 0; t2 < g.T; ++t2) p.y_out[(size_t)t2 * d_model + g.c0 + tid] = __builtin_nanf("");
  };

  float qs = 1.f;  // scale of the q held in LDS (its RMS normalisation, applied to the products)
  for (int t = 0; t < g.T; ++t) {
    qs = 1.f;
    for (int c = tid; c < d_model; c += kWorkers) S.q[c] = p.q_in[(size_t)t * d_model + c];
    bar();
    if (p.q_prenorm) {
      float ss = 0.f;
      for (int c = tid; c < d_model; c += kWorkers) ss += S.q[c] * S.q[c];
      ss = wave_sum_dpp(ss);
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
      const char* k2base = (const char*)tab_k2[l] + (size_t)g.n0 * k2row;
      if (p.tr_q && w == 0)
        for (int c = tid; c < d_model; c += kWorkers) p.tr_q[trow * d_model + c] = S.q[c] * qs;
      if (tid < g.nown) S.h[tid] = 0.f;

      // ---------------- predictor: the streamers form chunk dots, all waves sum them
      for (int tile = 0; tile < g.ntile; ++tile) {
        bar();  // G1
        reduce_tile(g, S, tile, lane, wv, qs);
        bar();  // G2
      }

      const bool own = lane < g.nown;
      const float hj = own ? S.h[lane] : 0.f;
      const uint32_t lkey = (uint32_t)(t * g.L + l + 1);  // this layer's value of the LDS flags
      if (wv == 0) {
        // ---------------- exchange A: per-workgroup (mean, M2) -> theta
        const float mean_w = wave_sum_dpp(hj) / (float)g.nown;
        const float dv = own ? hj - mean_w : 0.f;
        const float m2_w = wave_sum_dpp(dv * dv);
        if (lane < kRepA) {
          uint64_t* dst = p.stats + (size_t)lane * p.stats_stride + w;
          put_tagged(dst, mean_w, tagA);
          put_tagged(dst + kRecRow, m2_w, tagA);
        }
        // every record's two words in one polling loop: the means of all
        // workgroups are contiguous, then their M2 values
        const uint64_t* src = fresh(p.stats + (size_t)(g.rep % kRepA) * p.stats_stride);
        constexpr int KA = 8;  // 4 records (G <= 256) x 2 words per lane
        const uint64_t* pa[KA];
#pragma unroll
        for (int k = 0; k < KA / 2; ++k) {
          const int gg = lane + 64 * k;
          pa[2 * k] = gg < G ? src + gg : nullptr;
          pa[2 * k + 1] = gg < G ? src + kRecRow + gg : nullptr;
        }
        float vals[KA];
        const bool ok = gather_tagged2<KA>(pa, tagA ^ S.poison, vals, p.hdr, S.fmark, S.spin_limit);
        // two passes over the records: the mean, then the squared deviations
        // about it (Chan et al.'s combination, written as two plain sums)
        float s1 = 0.f;
#pragma unroll
        for (int k = 0; k < KA / 2; ++k) s1 += ngk[k] > 0.f ? ngk[k] * vals[2 * k] : 0.f;  // no record: no term
        const float mu = wave_sum_dpp(s1) / (float)g.d_ff;
        float s2 = 0.f;
#pragma unroll
        for (int k = 0; k < KA / 2; ++k) {
          const float d = vals[2 * k] - mu;
          s2 += ngk[k] > 0.f ? vals[2 * k + 1] + ngk[k] * d * d : 0.f;
        }
        const float m2 = wave_sum_dpp(s2);
        const float theta = mu + sqrtf(m2 / (float)g.d_ff) * p.z;
        if (__builtin_amdgcn_ballot_w64(!ok) != 0 && lane == 0) {
          S.fail = 1;
          raise_failure(p.hdr, S.fmark);
        }
        if (lane == 0) {
          S.theta = theta;
          lds_signal(&S.aflag, lkey);
        }
        // ---------------- the selection mask goes out as soon as theta is
        // known; it is the word the readers of exchange B poll, and the gated
        // values follow from wave 1 once the candidates' K2 dots are done (a
        // reader that finds an entry without its tag polls it)
        const uint64_t M = __builtin_amdgcn_ballot_w64(own && hj > theta);
        if (lane < 2 * kRepB) {
          const int rp = lane >> 1;
          put_tagged_u32(p.rec + (size_t)rp * p.rec_stride + (size_t)(lane & 1) * kRecRow + w,
                         (lane & 1) ? (uint32_t)(M >> 32) : (uint32_t)M, tagB);
        }
      } else {
        // ---------------- waves 1..3, meanwhile: K2 dots of the top candidates.
        // Rank of each owned score among the workgroup's (ties by index), by
        // broadcasting every lane's score across the wave (no LDS traffic).
        int rank = 0;
        for (int i = 0; i < g.nown; ++i) {
          const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hj), i));
          rank += (hi > hj || (hi == hj && i < lane)) ? 1 : 0;
        }
        const bool isc = own && rank < kCand;
        const uint64_t cmask = __builtin_amdgcn_ballot_w64(isc);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(cmask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cmask, 0));
        // this wave's candidates: positions wv-1, wv+2, wv+5, wv+8 (those below
        // kCand), one per row of 16 lanes; a row without a candidate repeats
        // the wave's first row (its loads hit the caches) and stores nothing
        static_assert(kCand <= 12, "three waves of four 16-lane rows");
        int jsel[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint64_t bb = __builtin_amdgcn_ballot_w64(isc && pos == (wv - 1) + 3 * u);
          jsel[u] = bb ? __builtin_ctzll(bb) : -1;
        }
        if (jsel[0] >= 0) {
          const int grp = lane >> 4;
          const int jm = grp == 0 ? jsel[0] : grp == 1 ? jsel[1] : grp == 2 ? jsel[2] : jsel[3];
          const float d = k2_dot_row16<W>(k2base + (size_t)(jm >= 0 ? jm : jsel[0]) * k2row, S.q + g.r, g.K2C,
                                          lane & 15);
          if ((lane & 15) == 0 && jm >= 0) S.g[jm] = d * qs;
        }
        if (lane == 0) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __hip_atomic_fetch_add(&S.dotcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (wv == 1) {
          // ---------------- gated values of the selected neurons, published
          // once theta and every candidate's K2 dot are known
          const bool okw = lds_wait_ge(&S.dotcnt, 3 * lkey) && lds_wait_ge(&S.aflag, lkey);
          if (!okw && lane == 0) S.fail = 1;
          const float theta = S.theta;
          const bool on = own && hj > theta;
          const uint64_t M = __builtin_amdgcn_ballot_w64(on);
          uint64_t miss = M & ~cmask;
          while (miss) {  // selected neurons outside the candidates (rare)
            const int j = __builtin_ctzll(miss);
            miss &= miss - 1;
            const float d = k2_dot<W>(k2base + (size_t)j * k2row, S.q + g.r, g.K2C, lane);
            if (lane == 0) S.g[j] = d * qs;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          const float cval = on ? gelu_tanh(hj - theta) * S.g[lane < 64 ? lane : 0] : 0.f;
          const int e = __builtin_amdgcn_mbcnt_hi((uint32_t)(M >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)M, 0));
          if (on) {
            if (e < kRecEntries) {
#pragma unroll
              for (int rp = 0; rp < kRepB; ++rp)
                put_tagged(p.rec + (size_t)rp * p.rec_stride + (size_t)(2 + e) * kRecRow + w, cval, tagB);
            } else {
              put_tagged(p.ovf + (size_t)w * kOvfWords + (e - kRecEntries), cval, tagB);
            }
          }
        }
      }
      // ---------------- exchange B: every workgroup's selection mask (thread
      // tid polls record tid's two mask words; records are word-major, so one
      // load instruction of a wave reads the same word of 64 records from a
      // few cache lines).  The entries are read once, with their V rows, in
      // v_record.
      bool okB = true;
      uint64_t Mg = 0;
      if (tid < G) {
        const uint64_t* recm = fresh(p.rec + (size_t)(g.rep % kRepB) * p.rec_stride) + tid;
        const uint64_t* mp[2] = {recm, recm + kRecRow};
        float mv[2];
        okB = gather_tagged2<2>(mp, tagB, mv, p.hdr, S.fmark, S.spin_limit);
        if (okB) Mg = ((uint64_t)__float_as_uint(mv[1]) << 32) | __float_as_uint(mv[0]);
        S.cnt[tid] = okB ? __builtin_popcountll(Mg) : 0;
      }
      if (!okB) S.fail = 1;

      // ---------------- V: the owned columns of y.  Thread gg takes the
      // selected neurons of record gg; column sums then run over lanes and
      // waves in a fixed order.
      {
        const char* vbase = (const char*)tab_v[l] + (size_t)g.ch0 * 16;
        const uint64_t* recp = fresh(p.rec + (size_t)(g.rep % kRepB) * p.rec_stride) + (tid < G ? tid : 0);
        float acc[2 * CN];
#pragma unroll
        for (int i = 0; i < 2 * CN; ++i) acc[i] = 0.f;
        bool okV = true;
        if (tid < G && okB) {
          if (g.nch > 1)
            okV = v_record<W, 2>(p, S, vbase, vrow, Mg, nb_rec, recp, tid, tagB, acc);
          else
            okV = v_record<W, 1>(p, S, vbase, vrow, Mg, nb_rec, recp, tid, tagB, acc);
        }
        if (!okV) S.fail = 1;
        int col;
        if (g.nch > 1) {
          const float sum = wave_colsum<2 * CN>(acc, lane, col);
          if ((lane & (64 / (2 * CN) - 1)) == 0 && col < g.ncol) S.colpart[wv][col] = sum;
        } else {  // one owned chunk: only the first CN sums are needed
          float a1[CN];
#pragma unroll
          for (int i = 0; i < CN; ++i) a1[i] = acc[i];
          const float sum = wave_colsum<CN>(a1, lane, col);
          if ((lane & (64 / CN - 1)) == 0 && col < g.ncol) S.colpart[wv][col] = sum;
        }
      }

      // ---------------- trace (workgroup 0 only): the selected list in
      // ascending neuron order, its length and theta
      if (trace_here) {
        bar();  // T1
        if (wv == 0) {  // exclusive prefix of the counts, workgroup order
          int c4[4], s4 = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int gg = 4 * lane + k;
            c4[k] = gg < G ? S.cnt[gg] : 0;
            s4 += c4[k];
          }
          int run = wave_excl_scan(s4, lane);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int gg = 4 * lane + k;
            if (gg < G) S.off[gg] = run;
            run += c4[k];
          }
          if (lane == 63) S.ntot = run;
        }
        bar();  // T2
        if (tid < G && p.tr_idx) {
          const int n = __builtin_popcountll(Mg), o = S.off[tid];
          uint64_t mm = Mg;
          for (int e = 0; e < n; ++e) {
            const int j = __builtin_ctzll(mm);
            mm &= mm - 1;
            if (o + e < p.tr_cap) p.tr_idx[trow * p.tr_cap + o + e] = nb_rec + j;
          }
        }
        if (tid == 0) {
          if (p.tr_counts) p.tr_counts[trow] = S.ntot;
          if (p.tr_theta) p.tr_theta[trow] = S.theta;
        }
      }
      bar();  // V
      if (S.fail) {
        fail_out();
        return;
      }
      const float ymine =
          tid < g.ncol ? ((S.colpart[0][tid] + S.colpart[1][tid]) + S.colpart[2][tid]) + S.colpart[3][tid] : 0.f;
      if (last) {
        if (tid < g.ncol) p.y_out[(size_t)t * d_model + g.c0 + tid] = ymine;
        bar();  // Y
        continue;
      }

      // ---------------- exchange C: owned columns of y -> every workgroup, with
      // the sum of squares of the RMS normalisation taken on the way.  Thread
      // t gathers (and later scales) columns t, t + 256, ..., the same in
      // every workgroup, so every workgroup forms the same scale bit for bit.
      {
        if (tid < g.ncol)
#pragma unroll
          for (int rp = 0; rp < kRepC; ++rp) put_tagged(p.ycol + (size_t)rp * p.ycol_stride + g.c0 + tid, ymine, tagC);
        bool okC = true;
        float ss = 0.f;
        const uint64_t* src = fresh(p.ycol + (size_t)(g.rep % kRepC) * p.ycol_stride);
        constexpr int KC = 9;
        for (int c00 = 0; okC && c00 < d_model; c00 += kWorkers * KC) {
          const uint64_t* ptrs[KC];
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const int c = c00 + tid + kWorkers * k;
            ptrs[k] = c < d_model ? src + c : nullptr;
          }
          float vals[KC];
          okC = gather_tagged2<KC>(ptrs, tagC, vals, p.hdr, S.fmark, S.spin_limit);
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const int c = c00 + tid + kWorkers * k;
            if (c < d_model) {
              S.q[c] = vals[k];
              ss += vals[k] * vals[k];
            }
          }
        }
        ss = wave_sum_dpp(ss);
        if (lane == 0) S.wred[wv] = ss;
        if (!okC) S.fail = 1;
      }
      bar();  // C
      if (S.fail) {
        fail_out();
        return;
      }
      // the layer output stays in LDS as gathered; its RMS normalisation is the
      // scale qs applied to every product formed with it in the next layer
      qs = 1.f / sqrtf((S.wred[0] + S.wred[1] + S.wred[2] + S.wred[3]) / (float)d_model + p.eps);
    }
  }
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
  g.n0 = own_first(g.w, g.d_ff, g.G);
  g.nown = own_first(g.w + 1, g.d_ff, g.G) - g.n0;
  col_range(g.w, g.G, g.d_model, CN, g.c0, g.ncol);
  g.ch0 = g.c0 / CN;
  g.nch = g.ncol / CN;
  g.CK = g.r / CN;
  g.K2C = (g.d_model - g.r) / CN;
  g.TC = g.nown * g.CK;
  g.ntile = (g.TC + kStreamers * kDecMaxC - 1) / (kStreamers * kDecMaxC);
  g.rep = xcc_id() + 8 * ((g.w >> 3) & 1);
  if (threadIdx.x == 0) {
    S.tag0 = (uint32_t)get_word(p.hdr);
    S.fmark = (uint64_t)S.tag0 + 1;
    // hdr[3], when nonzero, is a host-set test hook that drives the failure
    // path: it replaces the bound of every wait, and exchange A waits for a
    // tag no word carries (bit 31 flipped: the statistics words hold this
    // layer's or the previous layer's tag), so every workgroup times out
    // there and every wave still exits
    const uint64_t lim = get_word(p.hdr + 3);
    S.spin_limit = lim ? (uint32_t)lim : p.spin_limit;
    S.poison = lim ? 0x80000000u : 0u;
    S.fail = 0;
    S.aflag = 0;
    S.dotcnt = 0;
  }
  __syncthreads();
  if (threadIdx.x < kWorkers) {
    decode_worker<W>(p, kp->k2t, kp->v, g, S);
    // on every way out, failed or not: the next call's tags start after the
    // T (3 L - 1) tags this call owns (A, B and C per layer, no C after the
    // last).  Every workgroup has read hdr[0] before it published anything,
    // and workgroup 0 cannot get past the first exchange before that.
    if (g.w == 0 && threadIdx.x == 0)
      __hip_atomic_store(p.hdr, (uint64_t)(S.tag0 + (uint32_t)g.T * (uint32_t)(3 * g.L - 1)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    decode_streamer<W>(p, kp->k1t, kp->v, g, S);
  }
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct DecodeLayout {
  size_t hdr, stats, rec, ovf, ycol, qbuf, total;
  int stats_stride, rec_stride, ycol_stride;
};

static DecodeLayout decode_layout(int64_t d_model, int64_t T, int grid, int n_layers) {
  DecodeLayout L;
  L.stats_stride = (int)round_up((size_t)2 * kRecRow + 64, 512);  // words; replicas 4 KB+ apart
  L.rec_stride = (int)round_up((size_t)kRecWords * kRecRow + 64, 512);
  L.ycol_stride = (int)round_up((size_t)d_model + 64, 512);
  size_t off = 0;
  L.hdr = off;
  off += 256;
  L.stats = off;
  off += round_up((size_t)kRepA * L.stats_stride * 8, 256);
  L.rec = off;
  off += round_up((size_t)kRepB * L.rec_stride * 8, 256);
  L.ovf = off;
  off += round_up((size_t)grid * kOvfWords * 8, 256);
  L.ycol = off;
  off += round_up((size_t)kRepC * L.ycol_stride * 8, 256);
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
  // the workgroups exchange data while they run, so the device must hold the
  // whole grid at once (one workgroup per compute unit)
  if ((int64_t)per_cu * device_cu_count() < grid) return hipErrorLaunchOutOfResources;
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
    p.rec = (uint64_t*)(base + Lo.rec);
    p.ovf = (uint64_t*)(base + Lo.ovf);
    p.ycol = (uint64_t*)(base + Lo.ycol);
    p.stats_stride = Lo.stats_stride;
    p.rec_stride = Lo.rec_stride;
    p.ycol_stride = Lo.ycol_stride;
    p.spin_limit = 1u << 22;
    void* args[] = {&p};
    // An ordinary launch: on a device that holds the grid every workgroup
    // starts at once (the cooperative launch API guarantees the same thing but
    // costs ~16-20 us more per call here).  Were other work to keep some
    // workgroups from starting, the bounded waits would end the call as a
    // recorded failure, never a hang.
    e = hipLaunchKernel((const void*)decode_kernel<W>, dim3(grid), dim3(kDecodeThreads), args, 0, st);
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

// ---------------------------------------------------------------- no-allocation variant
// The workspace of spark_ffn_decode_noalloc: one array per device, kept for the
// life of the process, shared by every call on that device (it carries the
// exchange tags from call to call like a caller's workspace).  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static __global__ void zero_words(uint64_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

namespace {
struct NoAllocDevice {
  void* ptr = nullptr;    // device address of `scratch` on this device
  uint64_t tags = 0;      // exchange tags used since the scratch was last cleared
  bool cleared = false;   // the first clear has been enqueued
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kMaxDevices];
}  // namespace

hipError_t launch_decode_noalloc(const spark_ffn_shape& s, const spark_ffn_weights* layers, int n_layers,
                                 const float* q, int64_t T, float* y, float eps, double z,
                                 const spark_ffn_trace* trace, uint64_t tags, hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> g(g_noalloc_mu);
    NoAllocDevice& d = g_noalloc[dev];
    if (!d.ptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      d.ptr = p;
    }
    // clear before the first call on this device, and again before the 32-bit
    // tags would wrap (a tag must never repeat while a word can carry it)
    if (!d.cleared || d.tags + tags > 0xFFFFFFFFull) {
      const size_t words = kNoAllocScratchBytes / 8;
      hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, st, (uint64_t*)d.ptr, words);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      d.cleared = true;
      d.tags = 0;
    }
    d.tags += tags;
    ws = d.ptr;
  }
  return launch_decode(s, layers, n_layers, q, T, y, eps, z, trace, ws, st);
}

}  // namespace spark
