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
#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"
#include "internal.hpp"

namespace spark {

// z[n] = Q(1 - k/n) for n in (k, T] (0 elsewhere), in fp64: the tail
// probability P(Z > w) = tt is solved from the rational approximation of
// Abramowitz and Stegun 26.2.23 (error below 4.5e-4) by Newton steps on
// erfc(w / sqrt 2) / 2 = tt, which converge monotonically (the tail is convex
// for w >= 0) and reach double precision in three.
__device__ __forceinline__ void z_entry(int k, int n, float* __restrict__ z) {
  if (n <= k) {
    z[n] = 0.f;
    return;
  }
  const double t = (double)k / (double)n;
  const bool upper = 2 * k <= n;
  const double tt = upper ? t : 1.0 - t;  // solve P(Z > w) = tt for w >= 0
  const double u = sqrt(-2.0 * log(tt));
  double w = u - (2.515517 + u * (0.802853 + u * 0.010328)) / (1.0 + u * (1.432788 + u * (0.189269 + u * 0.001308)));
  w = fmax(w, 0.0);
  for (int i = 0; i < 4; ++i) {
    const double pdf = 0.3989422804014327 * exp(-0.5 * w * w);
    if (!(pdf > 0.0)) break;
    w += (0.5 * erfc(w * 0.7071067811865476) - tt) / pdf;
  }
  z[n] = (float)(upper ? w : -w);
}
__global__ void z_table(int k, int T, float* __restrict__ z) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n <= T) z_entry(k, n, z);
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
                                                         int32_t* __restrict__ counts, float* __restrict__ theta,
                                                         uint32_t* __restrict__ sel, int nw) {
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
  if (sel) {
    // selection bitmask of the row (see sel_to_list): position j = 4 (tid + 256 c) + e
    // is bit j % 32 of word j / 32; the eight threads of a word OR their nibbles
    uint32_t* srow = sel + ((size_t)t * Hq + h) * nw;
#pragma unroll
    for (int c4 = 0; c4 < PER / 4; ++c4) {
      uint32_t nib = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) nib |= (ok[4 * c4 + e] && v[4 * c4 + e] > th) ? 1u << e : 0u;
      uint32_t wd = nib << (4 * (tid & 7));
      wd |= __shfl_xor(wd, 1, kWave);
      wd |= __shfl_xor(wd, 2, kWave);
      wd |= __shfl_xor(wd, 4, kWave);
      const int wi = (tid >> 3) + 32 * c4;
      if ((tid & 7) == 0 && 32 * wi < n) srow[wi] = wd;
    }
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

// Selected lists from the selection bitmasks: row (t, h) of sel holds bit
// j % 32 of word j / 32 set when position j <= t is attended.  One wave per
// row: words in rounds of 64 (one per lane), their popcounts scanned across
// the wave, each lane then writes the positions of its word's set bits in
// ascending order; the first min(count, cap) positions are stored and the
// rest of the row's cap slots read -1.
__global__ __launch_bounds__(256) void sel_to_list(const uint32_t* __restrict__ sel, int nw, int T, int Hq,
                                                   int32_t* __restrict__ idx, int64_t cap) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)T * Hq) return;
  const int t = (int)(row / Hq);
  const uint32_t* srow = sel + row * nw;
  int32_t* irow = idx + row * cap;
  const int nwr = t / 32 + 1;  // words holding positions 0..t
  int64_t base = 0;
  for (int w0 = 0; w0 < nwr; w0 += 64) {
    const int w = w0 + lane;
    uint32_t bits = w < nwr ? srow[w] : 0u;
    if (w == nwr - 1 && (t & 31) != 31) bits &= (1u << ((t & 31) + 1)) - 1u;  // positions past t
    const int pc = __builtin_popcount(bits);
    const int incl = wave_incl_scan_dpp(pc);
    const int64_t off = base + incl - pc;
    int e = 0;
    while (bits) {
      const int b = __builtin_ctz(bits);
      bits &= bits - 1;
      if (off + e < cap) irow[off + e] = 32 * w + b;
      ++e;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  for (int64_t e = base + lane; e < cap; e += 64) irow[e] = -1;
}

// ---------------------------------------------------------------- fused path
// The same operator without materialising any T x T array, for head shapes
// with r = hd - r in {32, 64, 128}.  Two kernels, both passes over the
// keys of each query on the matrix cores:
//   attn_prefill_moments: the scores s_j = q[:r].k1_j, tile by tile, reduced
//       to the count, mean and M2 of the row (Chan's pairwise merge) and its
//       maximum M; theta = mean + std * z(t + 1), -inf when t + 1 <= k_attn.
//   attn_prefill_fused: the scores again and the gate products q[r:].k2_j;
//       e_j = e^(s_j - M) on the selected j, l = sum of e_j,
//       O = sum of e_j softplus(.) v_j; out = O / l.
// Whenever a row selects anything its maximum is selected, so M is the
// largest selected score and no rescaling is needed while O accumulates.
//
// Work split.  Products are transposed, S^T = K1 Q^T (keys x queries), so the
// 32x32 MFMA result holds one query per lane and, with the rows of the key
// tile permuted (bits 2 and 3 of the row index swapped), register i of lane
// half hl holds key 16 (i / 8) + 8 hl + i % 8: eight consecutive keys per
// register half, which is the operand layout O^T += V^T P^T needs, straight
// from registers.  A workgroup holds two sets of 32 query rows that share one
// KV head (two heads of a group over the same queries, or 64 consecutive
// queries of one head); its waves split each step's key tiles between them
// and merge through LDS at the end of a phase.  Each workgroup takes query
// block i (walking its key tiles up from 0) and then the causal mirror block
// nq - 1 - i (walking down from its diagonal): every workgroup has the same
// number of tiles, and at any step the workgroups reading one KV head are on
// the same few tiles, which stay in the XCD's L2 (the workgroups of one KV
// head share an XCD).
namespace {

constexpr int kFusedThreads = 256;
constexpr int kMomentThreads = 512;
constexpr int kFusedThreads2 = 512;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS row of key row x of a tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int tile_perm(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

struct FusedArgs {
  const bf16_t* q;     // [T][Hq][hd]
  const bf16_t* k1;    // [Hkv][T][r]
  const bf16_t* k2;    // [Hkv][T][hd - r]
  const bf16_t* vt;    // [Hkv][hd][LT], zero past T
  const float* ztab;   // [T + 1]
  float* rth;          // [Hq][T] threshold (-inf: every position attended)
  float* rmx;          // [Hq][T] largest score of the row
  float* out;          // [T][Hq][hd]
  int32_t* counts;     // [T][Hq] or null
  float* theta;        // [T][Hq] or null
  uint8_t* sel;        // [T][Hq][selb] selection bitmask bytes (see sel_to_list), or null
  int selb;            // bytes per row of sel
  int T, Hq, G, LT, k_attn;
  int pair_heads;      // 1: the two row sets are heads 2u, 2u + 1 over 32 queries; 0: head u over 64 queries
  int nunits, nq;      // head pairs (or heads); query blocks of 32 (or 64) positions
};

// Rows and key tiles of one phase of a workgroup.
struct Phase {
  int q0[2], h[2];  // first query and head of each row set
  int last;         // last key tile any row of the phase needs
  bool down;        // tiles walked from `last` down to 0
  // tile p of step s with NTS tiles per step, and the number of steps
  template <int NTS>
  __device__ __forceinline__ int tile(int s, int p) const { return down ? last - NTS * s - p : NTS * s + p; }
  template <int NTS>
  __device__ __forceinline__ int steps() const { return last / NTS + 1; }
  // selects rather than indexing, which would put the arrays in scratch memory
  __device__ __forceinline__ int first(int r) const { return r ? q0[1] : q0[0]; }
  __device__ __forceinline__ int head(int r) const { return r ? h[1] : h[0]; }
};

__device__ __forceinline__ bool make_phase(const FusedArgs& a, int ph, Phase& P) {
  const int unit = blockIdx.x % a.nunits, task = blockIdx.x / a.nunits;
  const int qb = ph == 0 ? task : a.nq - 1 - task;
  if (ph == 1 && qb <= task) return false;
  if (a.pair_heads) {
    P.q0[0] = P.q0[1] = 32 * qb;
    P.h[0] = 2 * unit;
    P.h[1] = 2 * unit + 1;
  } else {
    P.q0[0] = 64 * qb;
    P.q0[1] = 64 * qb + 32;
    P.h[0] = P.h[1] = unit;
  }
  P.last = (P.q0[1] < a.T ? P.q0[1] : P.q0[0]) >> 5;
  P.down = ph == 1;
  return true;
}

// LDS of one step of the fused kernel: two key tiles of K1 and K2 (32 rows of
// R or RC bf16 plus a 16-byte pad) and two V^T tiles (HD rows of 32 keys, the
// four 16-byte chunks of row d stored in the order c ^ ((d / 4) % 4) so that
// sixteen consecutive rows read at one chunk hit sixteen bank groups), each
// region a whole number of 1 KB load jobs (64 lanes x 16 bytes).
template <int R, int RC>
struct FusedLds {
  static constexpr int HD = R + RC;
  static constexpr int K1S = R + 8, K2S = RC + 8, OS = HD + 4;  // row lengths
  static constexpr int J1 = R / 8 + 1, J2 = RC / 8 + 1, JV = HD / 8;
  static constexpr int K2_OFF = 1024 * J1, V_OFF = 1024 * (J1 + J2), BUF_BYTES = 1024 * (J1 + J2 + JV);
  static constexpr int O_BYTES = 4 * 2 * 32 * OS;
  static_assert(2 * 32 * K1S * 2 == 1024 * J1 && 2 * 32 * K2S * 2 == 1024 * J2 && 2 * HD * 64 == 1024 * JV,
                "regions are whole jobs");
  static_assert(O_BYTES <= BUF_BYTES, "output staging fits one tile buffer");
  static_assert(R == RC && K1S == K2S, "the score and gate chains of a wave pair have one shape");
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Raw buffer descriptor over `bytes` bytes from p (stride 0; word 3 as the
// gfx9 raw buffers take it): offsets at or past `bytes` read as zeros.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return rsrc_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
// 16 bytes per lane from byte offset voff of the buffer into LDS at
// lds + 16 * lane (lds is the same for the whole wave; M0 carries it, one wait
// state before the load reads it).  Written as inline assembly so that the
// compiler does not order the following LDS reads of the other buffer after
// it; the step loop waits for these loads (vmcnt) and synchronises before any
// wave reads what they wrote.  The instruction writes no register.
// (M0 is named as clobbered; the compiler keeps nothing in it in these kernels.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const rsrc_t& r, void* lds, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0): every load this wave issued, LDS-destination loads
// included, has landed.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Byte offset at step 0 of the 16-byte chunk lane `lane` of key job j moves
// (rows of W bf16): slot 64 j + lane of the two padded tiles; a pad slot
// re-reads chunk 0 of its row.
template <int W>
__device__ __forceinline__ int key_job_offset(int j, int lane, const Phase& F) {
  constexpr int NS = W / 8 + 1;
  const int S = 64 * j + lane, ts = S / (32 * NS), rem = S % (32 * NS), rr = rem / NS, p = rem % NS;
  const int key = 32 * (F.down ? F.last - ts : ts) + tile_perm(rr);
  return key * 2 * W + 16 * (p < W / 8 ? p : 0);
}
// V^T jobs (rows of LT bf16): lane `lane` of job j moves chunk
// (lane % 4) ^ ((lane / 16) % 4) of row 16 (j % (HD / 16)) + lane / 4 of tile
// slot j / (HD / 16): the lane part of its byte offset, and the job part at
// step 0 (the tile moves by 64 bytes per tile).
__device__ __forceinline__ int vt_lane_offset(int lane, int LT) {
  return (lane >> 2) * 2 * LT + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
}
template <int HD>
__device__ __forceinline__ int vt_job_offset(int j, const Phase& F, int LT) {
  const int ts = j / (HD / 16), jr = j % (HD / 16);
  return 32 * jr * LT + 64 * (F.down ? F.last - ts : ts);
}

// S^T tile (32 keys x 32 queries) from an LDS key tile and the query fragments.
template <int KS>
__device__ __forceinline__ f32x16 tile_scores(const bf16_t* tile, int ld, const bf16x8 (&qf)[KS], int col, int hl) {
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const bf16_t* p = tile + col * ld + 8 * hl;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(p + 16 * ks), qf[ks], acc, 0, 0,
                                                  0);
  return acc;
}

template <int KS>
__device__ __forceinline__ void load_qfrag(bf16x8 (&qf)[KS], const bf16_t* qrow) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, load16(qrow + 16 * ks));
}

// softplus(g) = max(g, 0) + log1p(e) with e = e^-|g|: log1p(e) as
// ln 2 * log2(1 + e) while e >= e^-8 (the rounding of 1 + e then costs at
// most 2e-4 of the result) and e itself below (the dropped -e^2/2 is under
// 2e-4 of it): two transcendental instructions.
__device__ __forceinline__ float softplus_gate(float g) {
  const float a = fabsf(g);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * a);
  const float l = a > 8.f ? e : 0.6931471805599453f * __builtin_amdgcn_logf(1.f + e);
  return (g > 0.f ? g : 0.f) + l;
}

}  // namespace

// Pass 1: per row the threshold and the largest score.  Eight waves: the two
// row sets times four key phases (tile 4 s + p of step s for phase p).  The
// four key tiles of a step go straight from memory to LDS (buffer loads with
// the LDS destination; keys outside the head read as zeros and are masked),
// double-buffered as in the fused kernel.
template <int R>
__global__ __launch_bounds__(kMomentThreads) void attn_prefill_moments(const FusedArgs a) {
  constexpr int KA = R / 16, K1S = R + 8;
  constexpr int JM = 2 * (R / 8 + 1);  // 1 KB load jobs per step: four padded tiles of 32 rows
  constexpr int NW = kMomentThreads / 64, NJ = (JM + NW - 1) / NW;
  constexpr int BUF = 1024 * JM;
  static_assert(4 * 32 * K1S * 2 == BUF, "four tiles are whole jobs");
  __shared__ alignas(16) char mb0[BUF];
  __shared__ alignas(16) char mb1[BUF];
  __shared__ float st[4][2][32][4];  // [phase][row set][query]: n, mean, M2, max
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = wv & 1, par = wv >> 1, col = lane & 31, hl = lane >> 5;
  const int T = a.T, Hq = a.Hq;
  for (int ph = 0; ph < 2; ++ph) {
    Phase F;
    if (!make_phase(a, ph, F)) break;
    const int h = F.head(rs), q0 = F.first(rs), diag = q0 >> 5, tq = q0 + col;
    const bool live = q0 < T;
    const int nsteps = F.steps<4>();
    const rsrc_t rk = make_rsrc(a.k1 + (size_t)(F.head(0) / a.G) * T * R, (uint32_t)T * R * 2);
    // this wave's jobs j = wv + NW i: per-lane byte offsets at step 0 (a step
    // moves the keys by 128)
    int o1[NJ];
#pragma unroll
    for (int i = 0; i < NJ; ++i) o1[i] = key_job_offset<R>(wv + NW * i, lane, F);
    const int dstep = (F.down ? -128 : 128) * 2 * R;
    auto issue = [&](char* buf, int s) {
#pragma unroll
      for (int i = 0; i < NJ; ++i)
        if (wv + NW * i < JM) load_lds16(rk, buf + 1024 * (wv + NW * i), (uint32_t)(o1[i] + s * dstep));
    };
    bf16x8 qa[KA];
    load_qfrag(qa, a.q + ((size_t)min(tq, T - 1) * Hq + h) * (2 * R) + 8 * hl);
    Moments mo = {0.f, 0.f, 0.f};
    float mx = -INFINITY;
    auto step = [&](const char* cur, char* nxt, int s) {
      wait_vmcnt0();
      __syncthreads();  // step s is in LDS; every wave is done with step s - 1
      if (s + 1 < nsteps) issue(nxt, s + 1);
      const int kt = F.tile<4>(s, par);
      if (live && kt >= 0 && kt <= diag) {
        const f32x16 sc = tile_scores<KA>(reinterpret_cast<const bf16_t*>(cur) + par * 32 * K1S, K1S, qa, col, hl);
        if (kt < diag) {
          // a whole tile: sixteen scores per lane
          float s0 = 0.f, s1 = 0.f, x0 = sc[0], x1 = sc[1];
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            s0 += sc[i];
            s1 += sc[i + 1];
            x0 = fmaxf(x0, sc[i]);
            x1 = fmaxf(x1, sc[i + 1]);
          }
          const float mt = (s0 + s1) * 0.0625f;
          float q0s = 0.f, q1s = 0.f;
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float d0 = sc[i] - mt, d1 = sc[i + 1] - mt;
            q0s = fmaf(d0, d0, q0s);
            q1s = fmaf(d1, d1, q1s);
          }
          const float n1 = mo.n + 16.f, f = 16.f * __builtin_amdgcn_rcpf(n1), d = mt - mo.mean;
          mo.mean = fmaf(d, f, mo.mean);
          mo.m2 = mo.m2 + (q0s + q1s) + d * d * mo.n * f;
          mo.n = n1;
          mx = fmaxf(mx, fmaxf(x0, x1));
        } else {
          // the diagonal tile: positions j <= t only
          float sum = 0.f, tmx = -INFINITY, c = 0.f;
          bool ok[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            ok[i] = 32 * kt + 16 * (i >> 3) + 8 * hl + (i & 7) <= tq;
            sum += ok[i] ? sc[i] : 0.f;
            tmx = ok[i] ? fmaxf(tmx, sc[i]) : tmx;
            c += ok[i] ? 1.f : 0.f;
          }
          if (c > 0.f) {
            Moments t;
            t.n = c;
            t.mean = sum / c;
            t.m2 = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float d = sc[i] - t.mean;
              t.m2 += ok[i] ? d * d : 0.f;
            }
            mo = merge(mo, t);
            mx = fmaxf(mx, tmx);
          }
        }
      }
    };
    wait_vmcnt0();  // the fragments above are in registers before the step loop
    issue(mb0, 0);
    for (int s = 0; s < nsteps; s += 2) {
      step(mb0, mb1, s);
      if (s + 1 < nsteps) step(mb1, mb0, s + 1);
    }
    __syncthreads();  // every wave is done with the tiles before the next phase's loads
    // the two lane halves hold the same query (lower half on the left)
    Moments o;
    o.n = __shfl_xor(mo.n, 32, kWave);
    o.mean = __shfl_xor(mo.mean, 32, kWave);
    o.m2 = __shfl_xor(mo.m2, 32, kWave);
    mo = hl == 0 ? merge(mo, o) : merge(o, mo);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (hl == 0) {
      st[par][rs][col][0] = mo.n;
      st[par][rs][col][1] = mo.mean;
      st[par][rs][col][2] = mo.m2;
      st[par][rs][col][3] = mx;
    }
    __syncthreads();
    if (par == 0 && hl == 0 && live && tq < T) {
      Moments m = {st[0][rs][col][0], st[0][rs][col][1], st[0][rs][col][2]};
      float x = st[0][rs][col][3];
#pragma unroll
      for (int p = 1; p < 4; ++p) {
        const Moments mp = {st[p][rs][col][0], st[p][rs][col][1], st[p][rs][col][2]};
        m = merge(m, mp);
        x = fmaxf(x, st[p][rs][col][3]);
      }
      const bool dense = tq + 1 <= a.k_attn;
      const float th = dense ? -INFINITY : m.mean + sqrtf(m.m2 / (float)(tq + 1)) * a.ztab[tq + 1];
      a.rth[(size_t)h * T + tq] = th;
      a.rmx[(size_t)h * T + tq] = x;
      if (a.theta) a.theta[(size_t)tq * Hq + h] = dense ? NAN : th;
    }
  }
}

// Pass 2: gated weights and O.  Eight waves: for each row set and key parity
// a pair of waves shares each tile: the lower one forms the scores on the
// matrix cores and from them the selection and e^(s - M), the upper one the
// gate products and their softplus; the two swap these (fp16, through LDS),
// both form the gated weights of the whole tile, and each accumulates O for
// half of the hd output dimensions (O needs every key of the tile).  Key and V^T tiles go
// straight from memory to LDS (buffer loads with the LDS destination, 16 bytes
// per lane; keys past the end of a head read as zeros), double-buffered: the
// loads of step s + 1 are in flight while step s computes.
template <int R, int RC>
__global__ __launch_bounds__(kFusedThreads2) void attn_prefill_fused(const FusedArgs a) {
  using L = FusedLds<R, RC>;
  constexpr int HD = L::HD, NB2 = HD / 64, KA = R / 16;
  constexpr int K1S = L::K1S, OS = L::OS;
  constexpr int J1 = L::J1, J2 = L::J2, JV = L::JV;  // 1 KB load jobs per step
  constexpr int NW = kFusedThreads2 / 64;
  constexpr float kL2E = 1.4426950408889634f;
  // two step buffers as separate LDS objects, so that the loads into one are
  // known not to alias the reads of the other
  __shared__ alignas(16) char buf0[L::BUF_BYTES];
  __shared__ alignas(16) char buf1[L::BUF_BYTES];
  __shared__ alignas(16) _Float16 xch[NW][64 * 16];  // per wave: e^(s - M) (lower) or the gates (upper)
  __shared__ float lc[2][2][2][32][2];            // [parity][half][row set][query]: l, count
  float* const om = reinterpret_cast<float*>(buf0);

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = wv & 1, par = (wv >> 1) & 1, half = wv >> 2, col = lane & 31, hl = lane >> 5;
  const int partner = wv ^ 4;
  const int T = a.T, Hq = a.Hq, LT = a.LT;
  const int vlane = vt_lane_offset(lane, LT);
  // V^T fragment address within a tile: row col of each 32-row block, chunk 2 ks + hl
  const int vfrag0 = col * 64 + 16 * ((hl) ^ ((col >> 2) & 3));
  const int vfrag1 = col * 64 + 16 * ((2 + hl) ^ ((col >> 2) & 3));

  for (int ph = 0; ph < 2; ++ph) {
    Phase F;
    if (!make_phase(a, ph, F)) break;
    const int h = F.head(rs), q0 = F.first(rs), diag = q0 >> 5, tq = q0 + col;
    const bool live = q0 < T;
    const int nsteps = F.steps<2>();
    const int g = F.head(0) / a.G;
    const rsrc_t r1 = make_rsrc(a.k1 + (size_t)g * T * R, (uint32_t)T * R * 2);
    const rsrc_t r2 = make_rsrc(a.k2 + (size_t)g * T * RC, (uint32_t)T * RC * 2);
    const rsrc_t rv = make_rsrc(a.vt + (size_t)g * HD * LT, (uint32_t)HD * LT * 2);
    // this wave's jobs: job j = wv + NW i of each region; per-lane byte
    // offsets at step 0 (a step moves the keys by 64)
    constexpr int N1 = (J1 + NW - 1) / NW, N2 = (J2 + NW - 1) / NW, NV = (JV + NW - 1) / NW;
    int o1[N1], o2[N2], ov[NV];
#pragma unroll
    for (int i = 0; i < N1; ++i) o1[i] = key_job_offset<R>(wv + NW * i, lane, F);
#pragma unroll
    for (int i = 0; i < N2; ++i) o2[i] = key_job_offset<RC>(wv + NW * i, lane, F);
#pragma unroll
    for (int i = 0; i < NV; ++i) ov[i] = vlane + vt_job_offset<HD>(wv + NW * i, F, LT);
    const int dir = F.down ? -1 : 1;
    auto issue = [&](char* buf, int s) {
      const int sk1 = s * dir * 128 * R, sk2 = s * dir * 128 * RC, svt = s * dir * 128;
      // a negative offset (a tile before the first) reads zeros
#pragma unroll
      for (int i = 0; i < N1; ++i)
        if (wv + NW * i < J1) load_lds16(r1, buf + 1024 * (wv + NW * i), (uint32_t)(o1[i] + sk1));
#pragma unroll
      for (int i = 0; i < N2; ++i)
        if (wv + NW * i < J2) load_lds16(r2, buf + L::K2_OFF + 1024 * (wv + NW * i), (uint32_t)(o2[i] + sk2));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (wv + NW * i < JV) load_lds16(rv, buf + L::V_OFF + 1024 * (wv + NW * i), (uint32_t)(ov[i] + svt));
    };

    // the lower wave of a pair holds q[:r] (scores), the upper one q[r:] (gates)
    bf16x8 qf[KA];
    load_qfrag(qf, a.q + ((size_t)min(tq, T - 1) * Hq + h) * HD + (half ? R : 0) + 8 * hl);
    float th = INFINITY, mxs = 0.f;
    if (live && tq < T) {
      th = a.rth[(size_t)h * T + tq];
      mxs = a.rmx[(size_t)h * T + tq] * kL2E;
    }
    f32x16 oacc[NB2];
#pragma unroll
    for (int b = 0; b < NB2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
    float lsum = 0.f;
    int cnt = 0;
    // step s: its tiles are in `cur`; the loads of step s + 1 go to `nxt`
    auto step = [&](const char* cur, char* nxt, int s) {
      wait_vmcnt0();
      __syncthreads();  // step s is in LDS; every wave is done with step s - 1
      if (s + 1 < nsteps) issue(nxt, s + 1);
      const int kt = F.tile<2>(s, par);
      const bool act = live && kt >= 0 && kt <= diag;
      if (act) {
        // S^T (lower wave) or G^T (upper wave) of the tile: register i of lane
        // half hl holds key 16 (i / 8) + 8 hl + i % 8; fragments read in pairs
        const bf16_t* kt_ = reinterpret_cast<const bf16_t*>(cur + (half ? L::K2_OFF : 0)) + par * 32 * K1S +
                            col * K1S + 8 * hl;
        // (one accumulation chain in K order: the order of tile_scores in the
        // moments pass, so both passes form the same scores bit for bit)
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int k0 = 0; k0 < KA; k0 += 2) {
          bf16x8 f[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) f[u] = *reinterpret_cast<const bf16x8*>(kt_ + 16 * (k0 + u));
#pragma unroll
          for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[u], qf[k0 + u], acc, 0, 0, 0);
        }
        f16x8 hv[2];
        if (half == 0) {
          auto exps = [&](auto dc) {
            constexpr bool DIAG = decltype(dc)::value;
            uint32_t bits = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = 32 * kt + 16 * (i >> 3) + 8 * hl + (i & 7);
              const bool sel = (!DIAG || key <= tq) && acc[i] > th;
              const float e = sel ? __builtin_amdgcn_exp2f(fmaf(acc[i], kL2E, -mxs)) : 0.f;
              lsum += e;
              cnt += sel ? 1 : 0;
              bits |= sel ? 1u << i : 0u;
              hv[i >> 3][i & 7] = (_Float16)e;
            }
            // keys 32 kt + 16 u + 8 hl + j: byte 4 kt + 2 u + hl of the row's bitmask
            if (a.sel && tq < T) {
              uint8_t* sb = a.sel + ((size_t)tq * Hq + h) * a.selb + 4 * kt + hl;
              sb[0] = (uint8_t)(bits & 0xFFu);
              sb[2] = (uint8_t)(bits >> 8);
            }
          };
          if (kt < diag)
            exps(std::integral_constant<bool, false>{});
          else
            exps(std::integral_constant<bool, true>{});
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) hv[i >> 3][i & 7] = (_Float16)softplus_gate(acc[i]);
        }
        *reinterpret_cast<f16x8*>(&xch[wv][16 * lane]) = hv[0];
        *reinterpret_cast<f16x8*>(&xch[wv][16 * lane + 8]) = hv[1];
      }
      __syncthreads();  // both halves of every pair are in LDS
      if (act) {
        // gated weights of the whole tile, the same in both waves of the pair
        // (the product of the same two fp16 values)
        bf16x8 pw[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f16x8 x = *reinterpret_cast<const f16x8*>(&xch[wv][16 * lane + 8 * u]);
          const f16x8 y = *reinterpret_cast<const f16x8*>(&xch[partner][16 * lane + 8 * u]);
#pragma unroll
          for (int j = 0; j < 8; ++j) pw[u][j] = (__bf16)((float)x[j] * (float)y[j]);
        }
        const char* vtt = cur + L::V_OFF + par * HD * 64 + half * (HD / 2) * 64;
#pragma unroll
        for (int b = 0; b < NB2; ++b) {
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(vtt + b * 2048 + vfrag0), pw[0], oacc[b], 0, 0, 0);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(vtt + b * 2048 + vfrag1), pw[1], oacc[b], 0, 0, 0);
        }
      }
    };
    wait_vmcnt0();  // the fragments above are in registers before the step loop
    issue(buf0, 0);
    for (int s = 0; s < nsteps; s += 2) {
      step(buf0, buf1, s);
      if (s + 1 < nsteps) step(buf1, buf0, s + 1);
    }
    lsum += __shfl_xor(lsum, 32, kWave);
    cnt += __shfl_xor(cnt, 32, kWave);
    __syncthreads();  // every wave is done with the tiles
    // O^T layout: lane l, register i of block b -> dim 32 b + 8 (i / 4) + 4 hl + i % 4, query col;
    // this wave holds dims half * HD / 2 ..
    float* orow = om + (rs * 32 + col) * OS + half * (HD / 2) + 4 * hl;
    if (par == 1) {
#pragma unroll
      for (int b = 0; b < NB2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(orow + 32 * b + 8 * j) = {oacc[b][4 * j], oacc[b][4 * j + 1],
                                                              oacc[b][4 * j + 2], oacc[b][4 * j + 3]};
    }
    if (hl == 0) {
      lc[par][half][rs][col][0] = lsum;
      lc[par][half][rs][col][1] = (float)cnt;
    }
    __syncthreads();
    if (par == 0) {
#pragma unroll
      for (int b = 0; b < NB2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4* p = reinterpret_cast<f32x4*>(orow + 32 * b + 8 * j);
          const f32x4 o = *p;
          *p = f32x4{oacc[b][4 * j], oacc[b][4 * j + 1], oacc[b][4 * j + 2], oacc[b][4 * j + 3]} + o;
        }
      if (half == 0 && hl == 0 && live && tq < T && a.counts)
        a.counts[(size_t)tq * Hq + h] = (int)(((lc[0][0][rs][col][1] + lc[0][1][rs][col][1]) +
                                               lc[1][0][rs][col][1]) + lc[1][1][rs][col][1]);
    }
    __syncthreads();
    // rows out, 16 bytes per thread per step, scaled by 1 / l
    constexpr int RCH = HD / 4;
#pragma unroll 4
    for (int c = tid; c < 2 * 32 * RCH; c += kFusedThreads2) {
      const int r2 = c / (32 * RCH), qq = (c / RCH) & 31, cc = c % RCH;
      const int t = F.first(r2) + qq;
      if (t >= T) continue;
      const float l = ((lc[0][0][r2][qq][0] + lc[0][1][r2][qq][0]) + lc[1][0][r2][qq][0]) + lc[1][1][r2][qq][0];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const f32x4 o = *reinterpret_cast<const f32x4*>(om + (r2 * 32 + qq) * OS + 4 * cc);
      *reinterpret_cast<f32x4*>(a.out + ((size_t)t * Hq + F.head(r2)) * HD + 4 * cc) = o * inv;
    }
    __syncthreads();  // the next phase's loads overwrite the output staging
  }
}

// vt[g][c][j] = v[g][j][c] for j < T and 0 for T <= j < LT, all KV heads in
// one launch: 64 x 64 tiles through LDS, 16-byte loads and stores.
// The last z-slice of the grid (blockIdx.z == Hkv) fills the threshold table
// z[0..T] instead (z_table's entries; the grid has at least 4 LT >= T + 1
// threads per slice), so the fused path needs no launch of its own for it.
__global__ __launch_bounds__(256) void transpose_v(const bf16_t* __restrict__ v, int T, int HD, int LT,
                                                   bf16_t* __restrict__ vt, int Hkv, int k, float* __restrict__ z) {
  __shared__ bf16_t tile[64][72];  // [key][dim]
  const int g = blockIdx.z, j0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
  if (g == Hkv) {
    const int n = (blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid;
    if (n <= T) z_entry(k, n, z);
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, key = e >> 3, cc = e & 7;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (j0 + key < T && c0 + 8 * cc < HD) x = load16(v + ((size_t)g * T + j0 + key) * HD + c0 + 8 * cc);
    *reinterpret_cast<u32x4*>(&tile[key][8 * cc]) = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, dim = e >> 3, kc = e & 7;
    if (c0 + dim < HD && j0 + 8 * kc < LT) {
      u32x4 x;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        x[w] = (uint32_t)tile[8 * kc + 2 * w][dim] | ((uint32_t)tile[8 * kc + 2 * w + 1][dim] << 16);
      *reinterpret_cast<u32x4*>(vt + ((size_t)g * HD + c0 + dim) * LT + j0 + 8 * kc) = x;
    }
  }
}

bool attn_prefill_fused_ok(int64_t hd, int64_t r) {
  return 2 * r == hd && (r == 32 || r == 64 || r == 128);
}

// ---------------------------------------------------------------- host side
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct AttnPrefillLayout {
  size_t S, W, Vt, rth, rmx, rl, z, sel, total;
};

// Words of one row of the selection bitmask.
static int64_t sel_words(int64_t T) { return (T + 31) / 32; }

static AttnPrefillLayout attn_prefill_layout(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, bool lists) {
  const int64_t LT = (T + 7) & ~(int64_t)7;
  const bool fused = attn_prefill_fused_ok(hd, r);
  AttnPrefillLayout L;
  size_t off = 0;
  L.S = off;  // fp32 scores [Hq][T][LT] (general path only)
  if (!fused) off += round_up((size_t)Hq * T * LT * 4, 256);
  L.W = off;  // bf16 gated weights [Hq][T][LT] (general path only)
  if (!fused) off += round_up((size_t)Hq * T * LT * 2, 256);
  L.Vt = off;  // bf16 V^T [Hkv][hd][LT]
  off += round_up((size_t)Hkv * hd * LT * 2, 256);
  L.rth = off;
  off += round_up((size_t)Hq * T * 4, 256);
  L.rmx = off;
  off += round_up((size_t)Hq * T * 4, 256);
  L.rl = off;
  if (!fused) off += round_up((size_t)Hq * T * 4, 256);
  L.z = off;
  off += round_up((size_t)(T + 1) * 4, 256);
  L.sel = off;  // selection bitmasks [T][Hq][sel_words(T)] (only when lists are asked for)
  if (lists) off += round_up((size_t)T * Hq * sel_words(T) * 4, 256);
  L.total = off;
  return L;
}

size_t attn_prefill_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, bool lists) {
  return attn_prefill_layout(T, Hq, Hkv, hd, r, lists).total;
}

template <int R>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t st) {
  const int grid = a.nunits * ((a.nq + 1) / 2);
  hipLaunchKernelGGL((attn_prefill_moments<R>), dim3((unsigned)grid), dim3(kMomentThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_prefill_fused<R, R>), dim3((unsigned)grid), dim3(kFusedThreads2), 0, st, a);
  return hipGetLastError();
}

static hipError_t attn_prefill_main(const void* q, const void* k1, const void* k2, const void* v, int64_t T,
                                    int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out,
                                    int32_t* counts, float* theta, uint32_t* sel, const AttnPrefillLayout& L, void* ws,
                                    hipStream_t st);

hipError_t launch_attn_prefill(const void* q, const void* k1, const void* k2, const void* v, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out, int32_t* counts,
                               int32_t* idx, int64_t cap, float* theta, void* ws, hipStream_t st) {
  const bool lists = idx != nullptr && cap > 0;
  const AttnPrefillLayout L = attn_prefill_layout(T, Hq, Hkv, hd, r, lists);
  uint32_t* sel = lists ? (uint32_t*)((char*)ws + L.sel) : nullptr;
  hipError_t e = attn_prefill_main(q, k1, k2, v, T, Hq, Hkv, hd, r, k_attn, out, counts, theta, sel, L, ws, st);
  if (e != hipSuccess || !lists) return e;
  const int64_t rows = T * Hq;
  hipLaunchKernelGGL(sel_to_list, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, (const uint32_t*)sel,
                     (int)sel_words(T), (int)T, (int)Hq, idx, cap);
  return hipGetLastError();
}

static hipError_t attn_prefill_main(const void* q, const void* k1, const void* k2, const void* v, int64_t T,
                                    int64_t Hq, int64_t Hkv, int64_t hd, int64_t r, int64_t k_attn, float* out,
                                    int32_t* counts, float* theta, uint32_t* sel, const AttnPrefillLayout& L, void* ws,
                                    hipStream_t st) {
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
  hipError_t e = hipSuccess;
  if (attn_prefill_fused_ok(hd, r)) {
    // V^T for the fused kernel, and (one more grid slice) the threshold table
    hipLaunchKernelGGL(transpose_v, dim3((unsigned)((LT + 63) / 64), (unsigned)((hd + 63) / 64), (unsigned)(Hkv + 1)),
                       dim3(256), 0, st, (const bf16_t*)v, Ti, D, LT, Vt, (int)Hkv, (int)k_attn, ztab);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    FusedArgs a;
    a.q = Q;
    a.k1 = (const bf16_t*)k1;
    a.k2 = (const bf16_t*)k2;
    a.vt = Vt;
    a.ztab = ztab;
    a.rth = rth;
    a.rmx = rmx;
    a.out = out;
    a.counts = counts;
    a.theta = theta;
    a.sel = (uint8_t*)sel;
    a.selb = (int)(4 * sel_words(T));
    a.T = Ti;
    a.Hq = H;
    a.G = G;
    a.LT = LT;
    a.k_attn = (int)k_attn;
    a.pair_heads = G % 2 == 0;
    a.nunits = a.pair_heads ? H / 2 : H;
    a.nq = a.pair_heads ? (Ti + 31) / 32 : (Ti + 63) / 64;
    switch (R) {
      case 32: return launch_fused_t<32>(a, st);
      case 64: return launch_fused_t<64>(a, st);
      default: return launch_fused_t<128>(a, st);
    }
  }
  // 0. the threshold table
  hipLaunchKernelGGL(z_table, dim3((unsigned)((T + 1 + 255) / 256)), dim3(256), 0, st, (int)k_attn, Ti, ztab);
  e = hipGetLastError();
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
                         theta, sel, (int)sel_words(T));
    else if (Ti <= 2048)
      hipLaunchKernelGGL(attn_prefill_rows<8>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta, sel, (int)sel_words(T));
    else if (Ti <= 4096)
      hipLaunchKernelGGL(attn_prefill_rows<16>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta, sel, (int)sel_words(T));
    else if (Ti <= 8192)
      hipLaunchKernelGGL(attn_prefill_rows<32>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta, sel, (int)sel_words(T));
    else
      hipLaunchKernelGGL(attn_prefill_rows<64>, g, b, 0, st, S, Ti, LT, H, (int)k_attn, ztab, rth, rmx, rl, counts,
                         theta, sel, (int)sel_words(T));
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
