// Dense bf16 GEMM on the matrix cores for the prefill paths, with the
// epilogues that apply the Spark gates.  Included by ffn_prefill.hip and
// attn_prefill.hip.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace spark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GBK = 64;       // K per LDS stage
constexpr int GLD = GBK + 8;  // LDS row length in bf16 (16-byte pad against bank conflicts)

enum { kEpiStore = 0, kEpiGate = 1, kEpiAttn = 2, kEpiStats = 3 };
enum { kCausalNone = 0, kCausalTiles = 1, kCausalK = 2 };

// Arguments of one (batched) product D = A * B^T.  Batch z = blockIdx.z uses
// A + z*sA, B + (z / bgroup)*sB, C + z*sC, H + z*sH and the row arrays + z*sR.
struct GemmArgs {
  const bf16_t* A;
  const bf16_t* B;
  void* C;
  int lda, ldb, ldc, M, N, K, ksplit, bgroup;
  int64_t sA, sB, sC;
  const float* H;  // fp32 scores read by the gate epilogues (row stride ldh)
  int ldh;
  int64_t sH;
  const float* r0;  // per-row arrays of the epilogues (see gemm_bf16_nt)
  const float* r1;
  const float* r2;
  int64_t sR;
  int causal;
  f32x4* stats;  // kEpiStats: per (row, wave column tile) {shift, sum, sum of squares}, [M][ceil(N / wave width)]
};

// Column sums over the 32 lanes of each half-wave of NV per-lane values, all
// at once (NV = 32): at each step a lane hands half the values it holds to
// its partner (lane xor m, m = 16, 8, 4, 2, 1) and adds the other half to what
// it receives; after the five steps lane l holds the full sum of value
// l mod 32 over its half.
__device__ __forceinline__ float half_colsum32(float (&v)[32], int lane) {
#pragma unroll
  for (int st = 0; st < 5; ++st) {
    const int m = 16 >> st, h = 16 >> st;
    const uint32_t upm = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + h]);
      const float give = __uint_as_float((a & upm) | (b & ~upm));
      const float keep = __uint_as_float((b & upm) | (a & ~upm));
      v[i] = keep + __shfl_xor(give, m, kWave);
    }
  }
  return v[0];
}

// D = A[M][K] (bf16, row stride lda) * B^T where B is stored [N][K] (bf16,
// row stride ldb), with K a multiple of 8 and 16-byte aligned rows, over the
// K range of split blockIdx.y (ksplit columns each, a multiple of 64).  Rows of
// A and B past M and N are clamped on load and not stored; K past the end
// reads as zeros.
//
// Workgroup tile (WM*MI*32) x (WN*NI*32): WM x WN waves, each holding MI x NI
// accumulators of v_mfma_f32_32x32x16_bf16 (a 32*MI x 32*NI block).  A wave
// reads MI + NI fragments from LDS per 16 of K for MI*NI MFMAs, one step of
// 16 ahead of the MFMAs that use them.  K in stages of 64 through two LDS
// buffers: while the MFMAs of stage s run, stage s+1 (loaded into registers
// during stage s-1) is written to the other buffer and stage s+2 is loaded,
// both spread over the four steps of 16; one barrier per stage.  Tiles are
// dealt to the eight XCDs in contiguous runs (eight M tiles at a time down
// the N tiles), so the A and B panels a run shares stay in that XCD's L2.
//   kEpiStore: C[m][n] (fp32, row stride ldc) = D; with a K split, split s
//              writes its partial to C + s * M * ldc.
//   kEpiGate:  C[m][n] (bf16) = GELU(H - r0[m]) * D where H = H[m][n] > r0[m]
//              (theta), else 0.
//   kEpiAttn:  C[m][n] (bf16) = e^(H - r1[m]) / r2[m] * softplus(D) where
//              n <= m and H > r0[m] (theta, -inf when every token is
//              attended; r1 the largest selected score, r2 the sum of
//              e^(s - r1) over the selected), else 0.
//   kEpiStats: as kEpiStore (no K split), and for every row the sums of
//              (x - s) and (x - s)^2 over each wave's NI*32 columns, with the
//              shift s the row's value in the wave's first column (so the
//              moments keep their precision whatever the row's mean), to
//              stats[m][tn * WN + wn] = {s, sum, sum of squares}: the per-row
//              moments of the product in column tiles without reading it back.
// causal: kCausalTiles skips tiles wholly above the diagonal (n0 > m0 + BM - 1);
// kCausalK stops K at the end of the tile's rows (A's columns past the
// diagonal tile are never read).
template <int EPI, int WM, int WN, int MI, int NI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_nt(const GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * MI * 32, BN = WN * NI * 32;
  constexpr int CA = BM * GBK / 8 / NT, CB = BN * GBK / 8 / NT;  // 16-byte chunks per thread per stage
  static_assert(CA * NT * 8 == BM * GBK && CB * NT * 8 == BN * GBK, "tile must split evenly over threads");
  __shared__ alignas(16) bf16_t As[2][BM * GLD];
  __shared__ alignas(16) bf16_t Bs[2][BN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M = g.M, N = g.N;
  const int MT = (M + BM - 1) / BM, NTN = (N + BN - 1) / BN;
  // workgroups are dealt round-robin to the 8 XCDs (gridDim.x a multiple of
  // 8): XCD x takes the tile indices [x * per, (x + 1) * per), ordered eight
  // M tiles at a time down the N tiles
  int tm, tn;
  {
    const int tiles = MT * NTN, per = (tiles + 7) / 8;
    const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (t >= tiles) return;
    constexpr int GM = 8;
    const int grp = t / (GM * NTN), rem = t % (GM * NTN);
    const int gm = min(GM, MT - grp * GM);
    tm = grp * GM + rem % gm;
    tn = rem / gm;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal == kCausalTiles && n0 > m0 + BM - 1) return;
  const int wm = wv / WN, wn = wv % WN;
  const int z = blockIdx.z;
  const bf16_t* A = g.A + (size_t)z * g.sA;
  const bf16_t* B = g.B + (size_t)(z / g.bgroup) * g.sB;
  const int lda = g.lda, ldb = g.ldb;
  const int kbeg = blockIdx.y * g.ksplit;
  int kend = min(g.K, kbeg + g.ksplit);
  if (g.causal == kCausalK) kend = min(kend, m0 + BM);
  const int KT = kend > kbeg ? (kend - kbeg + GBK - 1) / GBK : 0;

  // Two register sets of staged 16-byte chunks (stage s in set s & 1).
  // Chunk i of a stage belongs to step i % 4 of the stage that moves it.
  // Chunks past K are loaded from column 0 and zeroed when stored to LDS.
  // (chunk i moves in step i % 4: any count works; multiples of 4 keep the
  // four steps even)
  u32x4 ra[2][CA], rb[2][CB];
  auto gload_part = [&](int set, int k0, int part) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      if (i % 4 != part) continue;
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const int k = k0 + kc * 8;
      ra[set][i] = load16(A + (size_t)min(m0 + row, M - 1) * lda + (k < kend ? k : 0));
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (i % 4 != part) continue;
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const int k = k0 + kc * 8;
      rb[set][i] = load16(B + (size_t)min(n0 + row, N - 1) * ldb + (k < kend ? k : 0));
    }
  };
  auto sstore_part = [&](int set, int buf, int k0, int part) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      if (i % 4 != part) continue;
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const uint32_t keep = k0 + kc * 8 < kend ? ~0u : 0u;
      *reinterpret_cast<u32x4*>(&As[buf][row * GLD + kc * 8]) = ra[set][i] & keep;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (i % 4 != part) continue;
      const int c = tid + NT * i, row = c >> 3, kc = c & 7;
      const uint32_t keep = k0 + kc * 8 < kend ? ~0u : 0u;
      *reinterpret_cast<u32x4*>(&Bs[buf][row * GLD + kc * 8]) = rb[set][i] & keep;
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (KT > 0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) gload_part(0, kbeg, p);
#pragma unroll
    for (int p = 0; p < 4; ++p) gload_part(1, kbeg + min(1, KT - 1) * GBK, p);
#pragma unroll
    for (int p = 0; p < 4; ++p) sstore_part(0, 0, kbeg, p);
  }
  __syncthreads();
  const int ro = lane & 31, kh = (lane >> 5) * 8;  // lanes 0-31: k 0..7 of a step, lanes 32-63: k 8..15
  // One stage; its register set and LDS buffer (kt & 1) are compile-time
  // constants (the stage loop is unrolled by two).  Past the last stage the
  // last one is loaded and stored again (never read).
  auto stage = [&](auto setc, int kt) {
    constexpr int set = decltype(setc)::value, buf = set;
    const int k1 = kbeg + min(kt + 1, KT - 1) * GBK, k2 = kbeg + min(kt + 2, KT - 1) * GBK;
    bf16x8 a[2][MI], b[2][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[0][i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * MI * 32 + i * 32 + ro) * GLD + kh]);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      b[0][j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * NI * 32 + j * 32 + ro) * GLD + kh]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int cur = st & 1;
      if (st < 3) {
        const int ko = (st + 1) * 16 + kh;
#pragma unroll
        for (int i = 0; i < MI; ++i)
          a[cur ^ 1][i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * MI * 32 + i * 32 + ro) * GLD + ko]);
#pragma unroll
        for (int j = 0; j < NI; ++j)
          b[cur ^ 1][j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * NI * 32 + j * 32 + ro) * GLD + ko]);
      }
      sstore_part(set ^ 1, buf ^ 1, k1, st);
      gload_part(set, k2, st);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < KT; kt += 2) {
    stage(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < KT) stage(std::integral_constant<int, 1>{}, kt + 1);
  }
  // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
  const int ldc = g.ldc;
  float* Cf = reinterpret_cast<float*>(g.C) + (size_t)z * g.sC + (size_t)blockIdx.y * M * ldc;
  bf16_t* Cb = reinterpret_cast<bf16_t*>(g.C) + (size_t)z * g.sC;
  const float* H = g.H + (size_t)z * g.sH;
  const float* R0 = g.r0 + (size_t)z * g.sR;
  const float* R1 = g.r1 + (size_t)z * g.sR;
  const float* R2 = g.r2 + (size_t)z * g.sR;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    float p0[16], p1[16], p2[16];
    if (EPI != kEpiStore) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = min(m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), M - 1);
        p0[r] = R0[m];
        if (EPI == kEpiAttn) {
          p1[r] = R1[m];
          p2[r] = __builtin_amdgcn_rcpf(R2[m]);  // one reciprocal per row of the block
        }
      }
    }
    // the scores of all NI blocks of this row of blocks, loaded before any
    // is used (one round trip per row of blocks, not one per block)
    float hvs[EPI != kEpiStore ? NI : 1][16];
    if (EPI != kEpiStore) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = min(n0 + wn * NI * 32 + j * 32 + (lane & 31), N - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          hvs[j][r] = H[(size_t)min(m, M - 1) * g.ldh + n];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * NI * 32 + j * 32 + (lane & 31);
      const float* hv = hvs[EPI != kEpiStore ? j : 0];
      // row of register r: mb + 8 (r / 4) + r % 4; one address per block,
      // constant row offsets per register; the gates are selects (the
      // arithmetic runs for every element, as a wave with any selected lane
      // would run it anyway)
      const int mb = m0 + wm * MI * 32 + i * 32 + 4 * (lane >> 5);
      float* frow = Cf + (size_t)mb * ldc + n;
      bf16_t* brow = Cb + (size_t)mb * ldc + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dm = 8 * (r >> 2) + (r & 3), m = mb + dm;
        const bool in = m < M && n < N;
        if (EPI == kEpiStore || EPI == kEpiStats) {
          if (in) frow[(size_t)dm * ldc] = acc[i][j][r];
        } else if (EPI == kEpiGate) {
          const float gv = gelu_tanh(hv[r] - p0[r]) * acc[i][j][r];
          const float c = hv[r] > p0[r] ? gv : 0.f;
          if (in) brow[(size_t)dm * ldc] = f32_to_bf16(c);
        } else {
          const float gv =
              __builtin_amdgcn_exp2f(1.4426950408889634f * (hv[r] - p1[r])) * p2[r] * softplus_fast(acc[i][j][r]);
          const float c = (n <= m && hv[r] > p0[r]) ? gv : 0.f;
          if (in) brow[(size_t)dm * ldc] = f32_to_bf16(c);
        }
      }
    }
    if constexpr (EPI == kEpiStats) {
      // register r of lane half hl is row 8 (r / 4) + 4 hl + r % 4 of the block
      const int nw0 = n0 + wn * NI * 32;
      const int cnt = min(max(N - nw0, 0), NI * 32);
      if (cnt > 0) {
        const int hl = lane >> 5;
        float v[32], sh[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc[i][0][r]), 0));
          const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc[i][0][r]), 32));
          sh[r] = hl ? s1 : s0;
          float t1 = 0.f, t2 = 0.f;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const float dv = nw0 + j * 32 + (lane & 31) < N ? acc[i][j][r] - sh[r] : 0.f;
            t1 += dv;
            t2 += dv * dv;
          }
          v[r] = t1;
          v[16 + r] = t2;
        }
        const float tot = half_colsum32(v, lane);
        // lane l of a half holds value l % 32: the sum of row l % 16 (l % 32 < 16)
        // or its sum of squares
        const int c = lane & 31, r = c & 15;
        const int m = m0 + wm * MI * 32 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (m < M) {
          const int nparts = (N + NI * 32 - 1) / (NI * 32);
          float* dst = reinterpret_cast<float*>(g.stats + (size_t)m * nparts + tn * WN + wn);
          float shr = sh[0];
#pragma unroll
          for (int k = 1; k < 16; ++k) shr = r == k ? sh[k] : shr;
          if (c < 16) {
            dst[0] = shr;
            dst[1] = tot;
          } else {
            dst[2] = tot;
          }
        }
      }
    }
  }
}

// Y[m][n] = sum over s < S of P[s][m][n] (fixed order), fp32 [M][N] planes.
static __global__ void sum_partials(const float* __restrict__ P, int S, int64_t plane, float* __restrict__ Y) {
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

// Vt[n][k] = V[k][n] for a bf16 [K][N] matrix (Vt rows ldo apart), 64x64
// tiles through LDS.
static __global__ __launch_bounds__(256) void transpose_bf16(const bf16_t* __restrict__ V, int K, int N,
                                                             bf16_t* __restrict__ Vt, int ldo) {
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
    if (n0 + r < N && k0 + c < K) Vt[(size_t)(n0 + r) * ldo + k0 + c] = tile[c][r];
  }
}

// The same for K and N multiples of 8: 16-byte loads along N and 16-byte
// stores along K.
static __global__ __launch_bounds__(256) void transpose_bf16_x8(const bf16_t* __restrict__ V, int K, int N,
                                                                bf16_t* __restrict__ Vt, int ldo) {
  __shared__ bf16_t tile[64][72];  // [k][n]
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, kr = e >> 3, cc = e & 7;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (k0 + kr < K && n0 + 8 * cc < N) x = load16(V + (size_t)(k0 + kr) * N + n0 + 8 * cc);
    *reinterpret_cast<u32x4*>(&tile[kr][8 * cc]) = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, nr = e >> 3, kc = e & 7;
    if (n0 + nr < N && k0 + 8 * kc < K) {
      u32x4 x;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        x[w] = (uint32_t)tile[8 * kc + 2 * w][nr] | ((uint32_t)tile[8 * kc + 2 * w + 1][nr] << 16);
      *reinterpret_cast<u32x4*>(Vt + (size_t)(n0 + nr) * ldo + k0 + 8 * kc) = x;
    }
  }
}

// Tile configurations of the prefill products.  General: 128 x 128 per
// workgroup, four waves of 64 x 64 (two workgroups per CU).  Large single
// products: 256 x 192, eight waves of 64 x 96 (one workgroup per CU, 126 KB of
// LDS; a wave reads five fragments per six MFMAs instead of four per four),
// used when its tiles times the K splits fill every CU at least once — at
// 4096 x 9216 that is 768 tiles, three full rounds (104 against 117 us for
// K = 1152); at 4096 x 2304 with four K splits, 768 workgroups.  (Two waves
// of 128 x 64, at one wave per SIMD, measured slower: too little to hide the
// LDS and global latencies; 256 x 256 and 192 x 256 tiles leave a partly
// filled last round at 4096 x 9216.)
constexpr int kWM = 2, kWN = 2, kMI = 2, kNI = 2;
constexpr int kBM = kWM * kMI * 32, kBN = kWN * kNI * 32;
constexpr int kWM2 = 4, kWN2 = 2, kMI2 = 2, kNI2 = 3;
constexpr int kBM2 = kWM2 * kMI2 * 32, kBN2 = kWN2 * kNI2 * 32;

// Whether launch_gemm takes the large 256 x 192 tiles for this product.
template <int EPI>
inline bool gemm_big_tiles(const GemmArgs& a, int splits, int batch) {
  if constexpr (EPI == kEpiAttn) return false;
  int cus = device_cu_count();
  if (cus < 1) cus = 256;
  const int64_t big = (int64_t)((a.M + kBM2 - 1) / kBM2) * ((a.N + kBN2 - 1) / kBN2);
  return batch == 1 && a.causal == kCausalNone && big * splits >= cus;
}

// Columns each wave of the chosen tile covers (the column tiles of kEpiStats).
template <int EPI>
inline int gemm_wave_cols(const GemmArgs& a, int splits, int batch) {
  return gemm_big_tiles<EPI>(a, splits, batch) ? kNI2 * 32 : kNI * 32;
}

// Launch over batch `batch` (grid z) and `splits` K splits (grid y).
template <int EPI>
inline hipError_t launch_gemm(GemmArgs a, int splits, int batch, hipStream_t st) {
  int ks = (a.K + splits - 1) / splits;
  a.ksplit = (ks + GBK - 1) / GBK * GBK;
  if (a.bgroup < 1) a.bgroup = 1;
  if constexpr (EPI != kEpiAttn) {
    if (gemm_big_tiles<EPI>(a, splits, batch)) {
      const int64_t big = (int64_t)((a.M + kBM2 - 1) / kBM2) * ((a.N + kBN2 - 1) / kBN2);
      const int grid = (int)((big + 7) / 8 * 8);  // a multiple of the XCD count (see gemm_bf16_nt)
      hipLaunchKernelGGL((gemm_bf16_nt<EPI, kWM2, kWN2, kMI2, kNI2>), dim3(grid, splits, 1), dim3(kWM2 * kWN2 * 64),
                         0, st, a);
      return hipGetLastError();
    }
  }
  const int tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  const int grid = (tiles + 7) / 8 * 8;  // a multiple of the XCD count (see gemm_bf16_nt)
  hipLaunchKernelGGL((gemm_bf16_nt<EPI, kWM, kWN, kMI, kNI>), dim3(grid, splits, batch), dim3(kWM * kWN * 64), 0,
                     st, a);
  return hipGetLastError();
}

// A GemmArgs with only the operands of a plain product set.
inline GemmArgs gemm_args(const bf16_t* A, int lda, const bf16_t* B, int ldb, void* C, int ldc, int M, int N, int K) {
  GemmArgs a{};
  a.A = A;
  a.B = B;
  a.C = C;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.M = M;
  a.N = N;
  a.K = K;
  a.bgroup = 1;
  a.causal = kCausalNone;
  return a;
}

}  // namespace spark
