// Exchange helpers of the persistent decode kernels: polling of tagged words
// (see put_tagged / get_word), the failure mark of a call, and the K2 dot of
// one neuron by one wave.
#pragma once

#include "common.hpp"

namespace spark {

// Poll up to K tagged words (a null pointer is skipped).  All loads of a round
// are issued together and re-issued until every tag matches.  Returns false on
// timeout, or when another workgroup has recorded a failure.
template <int K>
__device__ __forceinline__ bool gather_tagged(const uint64_t* const (&ptrs)[K], uint32_t tag, float (&out)[K],
                                              const uint64_t* hdr, uint64_t fmark, uint32_t spin_limit) {
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
    if ((spin & 1023) == 1023 && get_word(hdr + 1) == fmark) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// As gather_tagged, with two polling rounds in flight: the loads of the next
// round are issued before the words of the previous one are checked, so a
// word that appears just after a round was issued is seen about half a round
// trip later instead of a whole one.
template <int K>
__device__ __forceinline__ bool gather_tagged2(const uint64_t* const (&ptrs)[K], uint32_t tag, float (&out)[K],
                                               const uint64_t* hdr, uint64_t fmark, uint32_t spin_limit) {
  bool got[K];
#pragma unroll
  for (int k = 0; k < K; ++k) got[k] = ptrs[k] == nullptr;
  uint64_t a[K], b[K];
  auto issue = [&](uint64_t (&r)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (!got[k]) r[k] = get_word(ptrs[k]);
  };
  auto check = [&](const uint64_t (&r)[K]) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (!got[k]) {
        if ((uint32_t)(r[k] >> 32) == tag) {
          out[k] = __uint_as_float((uint32_t)r[k]);
          got[k] = true;
        } else {
          all = false;
        }
      }
    }
    return all;
  };
  issue(a);
  for (uint32_t spin = 0;; spin += 2) {
    issue(b);
    if (check(a)) return true;
    issue(a);
    if (check(b)) return true;
    if (spin > spin_limit) return false;
    if ((spin & 1022) == 1022 && get_word(hdr + 1) == fmark) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// A uniform pointer the compiler must treat as produced anew where this is
// called: per-thread addresses derived from it are then formed inside the
// layer loop instead of being hoisted out of it and held in registers.
template <typename T>
__device__ __forceinline__ T* fresh(T* ptr) {
  asm volatile("" : "+s"(ptr));
  return ptr;
}

// Record that the call whose first tag is tag0 failed: its mark tag0 + 1 (never
// 0, the value of a fresh header) goes to hdr[1], which the waits of the
// same call poll; the first workgroup to set the mark also counts the failed
// call in hdr[2], which the host can read.
__device__ __forceinline__ void raise_failure(uint64_t* hdr, uint64_t fmark) {
  const uint64_t old = __hip_atomic_exchange(hdr + 1, fmark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old != fmark) __hip_atomic_fetch_add(hdr + 2, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K2^T q[r:] for one owned neuron, by one wave (chunks strided over lanes).
template <typename W>
__device__ __forceinline__ float k2_dot(const char* row, const float* qr, int K2C, int lane) {
  constexpr int CN = Chunk<W>::N;
  float s = 0.f;
  for (int c0 = 0; c0 < K2C; c0 += 192) {
    u32x4 raw[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) raw[k] = load16(row + (size_t)min(c0 + lane + 64 * k, K2C - 1) * 16);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int cc = c0 + lane + 64 * k;
      float wf[CN];
      Chunk<W>::widen(raw[k], wf);
      const float* qq = qr + (cc < K2C ? cc : 0) * CN;
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < CN; ++e) a += wf[e] * qq[e];
      s += cc < K2C ? a : 0.f;
    }
  }
  return wave_sum_dpp(s);
}

}  // namespace spark
