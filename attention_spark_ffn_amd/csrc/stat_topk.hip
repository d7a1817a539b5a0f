// Statistical top-k over the rows of an fp32 matrix, one workgroup per row.
//
// Operator (Spark Transformer reading notes, section "方法详解 / 关键设计",
// item "Statistical Top-k"): theta = mean(x) + std(x) * Q(1 - k/d) with the
// population std, then the soft-threshold max{x - theta, 0}; the output lists
// the nonzeros (x_i > theta) in ascending index order with values x_i - theta.
//
// gfx950 mapping: the row is held in registers (lane t owns the 4 consecutive
// elements 4t + 4*NT*e, e < E, read with 16-byte loads, so each load
// instruction of the workgroup covers 4*NT contiguous floats).  Mean and
// sum of squared deviations are two exact passes over the registers, reduced
// with wave butterflies and a fixed-order sum across waves.  Compaction: per
// chunk e each lane counts its survivors (0..4), a wave prefix scan plus the
// per-wave totals in LDS give every survivor its ascending output slot.
// One HBM read of the row, writes only the survivors.
#include "common.hpp"
#include "internal.hpp"

namespace spark {

template <int NT, int E, bool VEC>
__global__ __launch_bounds__(NT) void stat_topk_kernel(const float* __restrict__ x, int64_t rows, int d, int64_t ldx,
                                                       float z, float* __restrict__ vals, int32_t* __restrict__ idx,
                                                       int64_t cap, int32_t* __restrict__ counts,
                                                       float* __restrict__ theta_out) {
  constexpr int NW = NT / kWave;
  __shared__ float red[NW];
  __shared__ int wtot[NW][E];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const float* xr = x + row * ldx;
    float v[E][4];
    bool ok[E][4];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i0 = 4 * tid + 4 * NT * e;
      if (VEC && i0 + 3 < d) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr + i0));
        v[e][0] = t.x; v[e][1] = t.y; v[e][2] = t.z; v[e][3] = t.w;
#pragma unroll
        for (int j = 0; j < 4; ++j) ok[e][j] = true;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ok[e][j] = i0 + j < d;
          v[e][j] = ok[e][j] ? xr[i0 + j] : 0.f;
        }
      }
    }
    // pass 1: mean
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) s += v[e][j];  // masked entries are 0
    s = wave_sum(s);
    __syncthreads();
    if (lane == 0) red[wv] = s;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    const float mean = tot / (float)d;
    // pass 2: sum of squared deviations
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dv = v[e][j] - mean;
        q += ok[e][j] ? dv * dv : 0.f;
      }
    q = wave_sum(q);
    __syncthreads();
    if (lane == 0) red[wv] = q;
    __syncthreads();
    float m2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) m2 += red[w];
    const float theta = mean + sqrtf(m2 / (float)d) * z;

    // survivors per (lane, chunk) and per-wave prefix
    int cnt[E], pre[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) c += (ok[e][j] && v[e][j] > theta) ? 1 : 0;
      cnt[e] = c;
      pre[e] = wave_excl_scan(c, lane);
      const int wt = __shfl(pre[e] + c, kWave - 1, kWave);
      if (lane == 0) wtot[wv][e] = wt;
    }
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int t = wtot[w][e];
        before += (w < wv) ? t : 0;
        all += t;
      }
      pre[e] += base + before;
      base += all;
    }
    total = base;
    if (idx != nullptr || vals != nullptr) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (cnt[e] == 0) continue;
        int pos = pre[e];
        const int i0 = 4 * tid + 4 * NT * e;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ok[e][j] && v[e][j] > theta) {
            if (pos < cap) {
              if (idx) idx[row * cap + pos] = i0 + j;
              if (vals) vals[row * cap + pos] = v[e][j] - theta;
            }
            ++pos;
          }
        }
      }
    }
    if (tid == 0) {
      counts[row] = total;
      if (theta_out) theta_out[row] = theta;
    }
    __syncthreads();
  }
}

template <int NT, int E>
static hipError_t launch_e(bool vec, const float* x, int64_t rows, int d, int64_t ldx, float z, float* vals,
                           int32_t* idx, int64_t cap, int32_t* counts, float* theta, hipStream_t st) {
  const int64_t grid = rows < (1 << 30) ? rows : (1 << 30);
  if (vec)
    hipLaunchKernelGGL((stat_topk_kernel<NT, E, true>), dim3((unsigned)grid), dim3(NT), 0, st, x, rows, d, ldx, z,
                       vals, idx, cap, counts, theta);
  else
    hipLaunchKernelGGL((stat_topk_kernel<NT, E, false>), dim3((unsigned)grid), dim3(NT), 0, st, x, rows, d, ldx, z,
                       vals, idx, cap, counts, theta);
  return hipGetLastError();
}

hipError_t launch_stat_topk(const float* x, int64_t rows, int64_t d, int64_t ldx, double z, float* vals, int32_t* idx,
                            int64_t cap, int32_t* counts, float* theta, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 4 == 0);
  const float zf = (float)z;
  const int di = (int)d;
  // rows up to 16384 elements: 256 threads (several rows resident per CU);
  // longer rows: 1024 threads.
  if (d <= 1024) return launch_e<256, 1>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 2048) return launch_e<256, 2>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 4096) return launch_e<256, 4>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 6144) return launch_e<256, 6>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 8192) return launch_e<256, 8>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 9216) return launch_e<256, 9>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 12288) return launch_e<256, 12>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 16384) return launch_e<256, 16>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  if (d <= 32768) return launch_e<1024, 8>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
  return launch_e<1024, 16>(vec, x, rows, di, ldx, zf, vals, idx, cap, counts, theta, st);
}

}  // namespace spark
