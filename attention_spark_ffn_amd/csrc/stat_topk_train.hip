// Training side of the statistical top-k: the Huber-smoothed operator and its
// gradient, one workgroup per row.
//
// Operator (Spark Transformer reading notes, section "方法详解 / 关键设计",
// item "Statistical Top-k"): theta = mean(x) + std(x) * Q(1 - k/d) with the
// population std; the notes state that with Huber smoothing the operator is
// continuously differentiable.  The smoothing used: the soft-threshold
// max{u, 0}, u = x - theta, becomes
//     h(u) = 0 (u <= 0),  u^2 / (2 delta) (0 < u < delta),  u - delta / 2 (u >= delta),
// whose slope is h'(u) = min(max(u / delta, 0), 1).
//   forward:  y_i = h(x_i - theta)                     (dense row, zero below theta)
//   backward: a_i = dy_i h'(x_i - theta), A = sum_i a_i,
//             dx_j = a_j - (A / d) (1 + z (x_j - mean) / std)
// (the second term is A times d theta / d x_j: d mean / d x_j = 1/d and
// d std / d x_j = (x_j - mean) / (d std); a row with zero spread has a = 0).
//
// gfx950 mapping: as the statistical top-k kernel, the row is held in
// registers (16-byte lanes, each load instruction of the workgroup covering
// 4*NT contiguous floats), mean and squared deviations are two exact passes
// reduced in a fixed order, and the result goes out with streaming stores:
// one HBM read of the row (two for the backward: x and dy) and one write.
#include "common.hpp"
#include "internal.hpp"
#include "rows.hpp"

namespace spark {

__device__ __forceinline__ float huber_relu(float u, float delta, float inv2d) {
  return u <= 0.f ? 0.f : (u < delta ? u * u * inv2d : u - 0.5f * delta);
}
__device__ __forceinline__ float huber_slope(float u, float inv_delta) {
  return fminf(fmaxf(u * inv_delta, 0.f), 1.f);
}

// mean and population std of a row in registers (padding entries are 0 and
// excluded from the squared deviations)
template <int NT, int E, bool EXACT>
__device__ __forceinline__ void row_stats(const float (&v)[E][4], int d, int tid, float* red0, float* red1,
                                          float& mean, float& sd) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) s += (v[e][0] + v[e][1]) + (v[e][2] + v[e][3]);
  mean = block_sum<NT / kWave>(s, red0) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dv = v[e][j] - mean;
      q += (EXACT || 4 * tid + 4 * NT * e + j < d) ? dv * dv : 0.f;
    }
  sd = sqrtf(block_sum<NT / kWave>(q, red1) / (float)d);
}

template <int NT, int E, bool VEC, bool EXACT>
__global__ __launch_bounds__(NT) void huber_forward_kernel(const float* __restrict__ x, int64_t rows, int d_arg,
                                                           float z, float delta, float* __restrict__ y,
                                                           float* __restrict__ theta_out) {
  __shared__ float red[2][NT / kWave];
  const float inv2d = 0.5f / delta;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    int tid = threadIdx.x, d = d_arg;
    asm volatile("" : "+v"(tid), "+s"(d));
    float v[E][4];
    load_row<NT, E, VEC, EXACT>(x + row * d, d, tid, v);
    float mean, sd;
    row_stats<NT, E, EXACT>(v, d, tid, red[0], red[1], mean, sd);
    const float theta = mean + sd * z;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[e][j] = huber_relu(v[e][j] - theta, delta, inv2d);
    store_row<NT, E, VEC, EXACT>(y + row * d, d, tid, v);
    if (theta_out && tid == 0) theta_out[row] = theta;
  }
}

template <int NT, int E, bool VEC, bool EXACT>
__global__ __launch_bounds__(NT) void huber_backward_kernel(const float* __restrict__ x, const float* __restrict__ dy,
                                                            int64_t rows, int d_arg, float z, float delta,
                                                            float* __restrict__ dx) {
  __shared__ float red[3][NT / kWave];
  const float inv_delta = 1.f / delta;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    int tid = threadIdx.x, d = d_arg;
    asm volatile("" : "+v"(tid), "+s"(d));
    float v[E][4], g[E][4];
    load_row<NT, E, VEC, EXACT>(x + row * d, d, tid, v);
    load_row<NT, E, VEC, EXACT>(dy + row * d, d, tid, g);
    float mean, sd;
    row_stats<NT, E, EXACT>(v, d, tid, red[0], red[1], mean, sd);
    const float theta = mean + sd * z;
    // a_i = dy_i h'(x_i - theta) (0 past the row end, where dy reads 0)
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g[e][j] *= huber_slope(v[e][j] - theta, inv_delta);
        s += g[e][j];
      }
    const float A = block_sum<NT / kWave>(s, red[2]);
    const float c1 = A / (float)d;
    const float c2 = sd > 0.f ? c1 * z / sd : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[e][j] = (g[e][j] - c1) - c2 * (v[e][j] - mean);
    store_row<NT, E, VEC, EXACT>(dx + row * d, d, tid, g);
  }
}

template <int NT, int E>
static hipError_t launch_train(bool vec, bool bwd, const float* x, const float* dy, int64_t rows, int d, float z,
                               float delta, float* out, float* theta, hipStream_t st) {
  const int64_t grid = rows < (1 << 30) ? rows : (1 << 30);
  const dim3 g((unsigned)grid), b(NT);
  const bool exact = vec && d == 4 * NT * E;
  if (!bwd) {
    if (exact)
      hipLaunchKernelGGL((huber_forward_kernel<NT, E, true, true>), g, b, 0, st, x, rows, d, z, delta, out, theta);
    else if (vec)
      hipLaunchKernelGGL((huber_forward_kernel<NT, E, true, false>), g, b, 0, st, x, rows, d, z, delta, out, theta);
    else
      hipLaunchKernelGGL((huber_forward_kernel<NT, E, false, false>), g, b, 0, st, x, rows, d, z, delta, out, theta);
  } else {
    if (exact)
      hipLaunchKernelGGL((huber_backward_kernel<NT, E, true, true>), g, b, 0, st, x, dy, rows, d, z, delta, out);
    else if (vec)
      hipLaunchKernelGGL((huber_backward_kernel<NT, E, true, false>), g, b, 0, st, x, dy, rows, d, z, delta, out);
    else
      hipLaunchKernelGGL((huber_backward_kernel<NT, E, false, false>), g, b, 0, st, x, dy, rows, d, z, delta, out);
  }
  return hipGetLastError();
}

hipError_t launch_stat_topk_huber(bool backward, const float* x, const float* dy, int64_t rows, int64_t d, double z,
                                  float delta, float* out, float* theta, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const auto al = [](const void* p) { return p == nullptr || (uintptr_t)p % 16 == 0; };
  const bool vec = d % 4 == 0 && al(x) && al(dy) && al(out);
  const float zf = (float)z;
  const int di = (int)d;
  if (d <= 1024) return launch_train<256, 1>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 2048) return launch_train<256, 2>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 4096) return launch_train<256, 4>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 8192) return launch_train<256, 8>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 9216) return launch_train<256, 9>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 16384) return launch_train<256, 16>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  if (d <= 32768) return launch_train<1024, 8>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
  return launch_train<1024, 16>(vec, backward, x, dy, rows, di, zf, delta, out, theta, st);
}

}  // namespace spark
