// Statistical top-k over the rows of an fp32 matrix, one workgroup per row.
//
// Operator (Spark Transformer reading notes, section "方法详解 / 关键设计",
// item "Statistical Top-k"): theta = mean(x) + std(x) * Q(1 - k/d) with the
// population std, then the soft-threshold max{x - theta, 0}; the output lists
// the nonzeros (x_i > theta) in ascending index order with values x_i - theta.
//
// gfx950 mapping: the row is held in registers (lane t owns the 4 consecutive
// elements 4t + 4*NT*e, e < E, read with 16-byte loads, so each load
// instruction of the workgroup covers 4*NT contiguous floats).  Mean and sum
// of squared deviations are two exact passes over the registers, reduced with
// DPP wave sums and a fixed-order sum across waves.  Compaction: each lane
// keeps a 4-bit survivor mask per chunk; a DPP prefix scan of the mask counts
// plus the per-wave totals give every survivor its ascending slot without a
// serial walk; the list is staged in LDS and written out with contiguous
// stores.  One HBM read of the row, writes only the survivors.
#include "common.hpp"
#include "internal.hpp"
#include "rows.hpp"

namespace spark {

constexpr int kStage = 2048;  // list entries of a row staged in LDS before the contiguous write-out

// Shared memory of one workgroup: per-wave partial sums (mean, then M2),
// per-(wave, chunk) survivor counts, and the staged list.  Each array is
// written once per row between two barriers, so a row needs no trailing
// barrier before the next one starts.
template <int NW, int E>
struct StatShared {
  float red[2][NW];
  int wtot[NW][E];
  int s_idx[kStage];
  float s_val[kStage];
};

// theta = mean + std * z of one row held in registers: two exact passes (the
// mean, then the squared deviations about it; entries past the row end are 0
// and left out of the second), each reduced with DPP wave sums and then the
// waves in a fixed order.
template <int NT, int E, bool EXACT>
__device__ __forceinline__ float row_theta(const float (&v)[E][4], int d, int tid, float z, float* red0,
                                           float* red1) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) s += (v[e][0] + v[e][1]) + (v[e][2] + v[e][3]);
  const float mean = block_sum<NT / kWave>(s, red0) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dv = v[e][j] - mean;
      q += (EXACT || 4 * tid + 4 * NT * e + j < d) ? dv * dv : 0.f;
    }
  const float m2 = block_sum<NT / kWave>(q, red1);
  return mean + sqrtf(m2 / (float)d) * z;
}

// Statistics, threshold and list of one row held in registers.  theta_in:
// the rows' thresholds when given (the statistics are then not formed).
template <int NT, int E, bool EXACT>
__device__ __forceinline__ void process_row(const float (&v)[E][4], int64_t row, int d, int tid, float z,
                                            float* __restrict__ vals, int32_t* __restrict__ idx, int64_t cap,
                                            int32_t* __restrict__ counts, float* __restrict__ theta_out,
                                            const float* __restrict__ theta_in, StatShared<NT / kWave, E>& S) {
  constexpr int NW = NT / kWave;
  const int lane = tid & (kWave - 1), wv = tid / kWave;
  const float theta = theta_in ? theta_in[row] : row_theta<NT, E, EXACT>(v, d, tid, z, S.red[0], S.red[1]);

  // survivors of chunk e as a 4-bit mask per lane.  Pass A publishes each
  // (wave, chunk) total; pass B forms the masks and their in-wave prefix scans
  // again (rather than holding them across the barrier), adds the totals of
  // the earlier chunks and waves, and places every survivor at its ascending
  // slot without a serial walk.
  auto survivors = [&](int e) {
    int m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m |= ((EXACT || 4 * tid + 4 * NT * e + j < d) && v[e][j] > theta) ? (1 << j) : 0;
    // opaque: later tests read the bits rather than keeping the compares
    asm volatile("" : "+v"(m));
    return m;
  };
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int incl = wave_incl_scan_dpp(__builtin_popcount(survivors(e)));
    if (lane == kWave - 1) S.wtot[wv][e] = incl;
  }
  __syncthreads();
  int base = 0;  // survivors of the chunks before e, all waves
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int before = 0, all = 0;
#pragma unroll(NW <= 4 ? NW : 1)
    for (int w = 0; w < NW; ++w) {
      const int t = S.wtot[w][e];
      before += (w < wv) ? t : 0;
      all += t;
    }
    if (idx != nullptr || vals != nullptr) {
      const int m = survivors(e);
      const int c = __builtin_popcount(m);
      const int pre = base + before + wave_incl_scan_dpp(c) - c;
      // slot of survivor (e, j): the chunk's prefix plus this lane's
      // survivors before it in the chunk
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (m & (1 << j)) {
          const int pos = pre + __builtin_popcount(m & ((1 << j) - 1));
          const int i = 4 * tid + 4 * NT * e + j;
          if (pos < kStage) {
            S.s_idx[pos] = i;
            S.s_val[pos] = v[e][j] - theta;
          } else if (pos < cap) {
            if (idx) idx[row * cap + pos] = i;
            if (vals) vals[row * cap + pos] = v[e][j] - theta;
          }
        }
    }
    base += all;
  }
  if (tid == 0) {
    counts[row] = base;
    if (theta_out) theta_out[row] = theta;
  }
  if (idx != nullptr || vals != nullptr) {
    __syncthreads();
    const int nst = (int)min((int64_t)min(base, kStage), cap);
    // streaming (nontemporal) stores: the lists are not read back here
    for (int i = tid; i < nst; i += NT) {
      if (idx) __builtin_nontemporal_store(S.s_idx[i], idx + row * cap + i);
      if (vals) __builtin_nontemporal_store(S.s_val[i], vals + row * cap + i);
    }
  } else if (theta_in) {
    // no statistics barriers precede the next row's counts: wait here until
    // every wave has read this row's
    __syncthreads();
  }
}

// One workgroup per row (rows strided by the grid).
template <int NT, int E, bool VEC, bool EXACT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 && E <= 9 ? 4 : 1)))
void stat_topk_kernel(const float* __restrict__ x, int64_t rows, int d_arg, int64_t ldx, float z,
                      float* __restrict__ vals, int32_t* __restrict__ idx, int64_t cap, int32_t* __restrict__ counts,
                      float* __restrict__ theta_out, const float* __restrict__ theta_in) {
  __shared__ StatShared<NT / kWave, E> S;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    // Opaque copies of the thread index and the row length: the element
    // indices and bounds tests derived from them are formed anew for every
    // row instead of being hoisted out of the loop and held in registers.
    int tid = threadIdx.x, d = d_arg;
    asm volatile("" : "+v"(tid), "+s"(d));
    float v[E][4];
    load_row<NT, E, VEC, EXACT>(x + row * ldx, d, tid, v);
    process_row<NT, E, EXACT>(v, row, d, tid, z, vals, idx, cap, counts, theta_out, theta_in, S);
  }
}

template <int NT, int E>
static hipError_t launch_e(bool vec, const float* x, int64_t rows, int d, int64_t ldx, float z, float* vals,
                           int32_t* idx, int64_t cap, int32_t* counts, float* theta, const float* theta_in,
                           hipStream_t st) {
  const int64_t grid = rows < (1 << 30) ? rows : (1 << 30);
  const dim3 g((unsigned)grid), b(NT);
  if (vec && d == 4 * NT * E)
    hipLaunchKernelGGL((stat_topk_kernel<NT, E, true, true>), g, b, 0, st, x, rows, d, ldx, z, vals, idx, cap, counts,
                       theta, theta_in);
  else if (vec)
    hipLaunchKernelGGL((stat_topk_kernel<NT, E, true, false>), g, b, 0, st, x, rows, d, ldx, z, vals, idx, cap,
                       counts, theta, theta_in);
  else
    hipLaunchKernelGGL((stat_topk_kernel<NT, E, false, false>), g, b, 0, st, x, rows, d, ldx, z, vals, idx, cap,
                       counts, theta, theta_in);
  return hipGetLastError();
}

hipError_t launch_stat_topk(const float* x, int64_t rows, int64_t d, int64_t ldx, double z, float* vals, int32_t* idx,
                            int64_t cap, int32_t* counts, float* theta, hipStream_t st, const float* theta_in) {
  if (rows == 0) return hipSuccess;
  const bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 4 == 0);
  const float zf = (float)z;
  const int di = (int)d;
  // rows up to 16384 elements: 256 threads (several rows resident per CU);
  // longer rows: 1024 threads.
  if (d <= 1024) return launch_e<256, 1>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 2048) return launch_e<256, 2>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 4096) return launch_e<256, 4>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 6144) return launch_e<256, 6>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 8192) return launch_e<256, 8>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 9216) return launch_e<256, 9>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 12288) return launch_e<256, 12>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 16384) return launch_e<256, 16>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  if (d <= 32768) return launch_e<1024, 8>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
  return launch_e<1024, 16>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, theta_in, st);
}

}  // namespace spark
