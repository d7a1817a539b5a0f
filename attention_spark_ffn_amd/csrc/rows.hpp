// Rows of an fp32 matrix held in registers by one workgroup: the layout the
// row-wise statistical top-k kernels share.
#pragma once

#include "common.hpp"

namespace spark {

// Lane t's elements 4t + 4*NT*e + j (e < E, j < 4) of one row, so that each
// 16-byte load instruction of the workgroup covers 4*NT contiguous floats.
// Entries past the row end are 0.  EXACT: d == 4*NT*E, no bounds tests; VEC:
// the row is 16-byte aligned (whole chunks are loaded as one vector).
template <int NT, int E, bool VEC, bool EXACT>
__device__ __forceinline__ void load_row(const float* xr, int d, int tid, float (&v)[E][4]) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i0 = 4 * tid + 4 * NT * e;
    if (EXACT || (VEC && i0 + 3 < d)) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr + i0));
      v[e][0] = t.x;
      v[e][1] = t.y;
      v[e][2] = t.z;
      v[e][3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[e][j] = i0 + j < d ? xr[i0 + j] : 0.f;
    }
  }
}

// The same layout stored back (streaming stores); entries past the row end
// are not written.
template <int NT, int E, bool VEC, bool EXACT>
__device__ __forceinline__ void store_row(float* yr, int d, int tid, const float (&v)[E][4]) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i0 = 4 * tid + 4 * NT * e;
    if (EXACT || (VEC && i0 + 3 < d)) {
      __builtin_nontemporal_store(f32x4{v[e][0], v[e][1], v[e][2], v[e][3]}, reinterpret_cast<f32x4*>(yr + i0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < d) yr[i0 + j] = v[e][j];
    }
  }
}

// Sum over the workgroup in a fixed order (DPP wave sums, then the waves in
// order through red[NW]); every thread gets the total.  One barrier: red
// must not be written again until every wave has passed a later barrier.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  v = wave_sum_dpp(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += red[w];
  return t;
}

}  // namespace spark
