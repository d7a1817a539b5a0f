// Device-side helpers shared by the gfx950 kernels of the Spark FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spark {

constexpr int kWave = 64;

// ---------------------------------------------------------------- element access
typedef uint16_t bf16_t;  // raw bf16 bit pattern
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// 16 bytes of weights widened to fp32: 8 bf16 or 4 fp32 values.
template <typename W>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const u32x4& raw, float* out) {
    out[0] = __uint_as_float(raw.x);
    out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z);
    out[3] = __uint_as_float(raw.w);
  }
};
template <>
struct Chunk<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const u32x4& raw, float* out) {
    out[0] = __uint_as_float(raw.x << 16);
    out[1] = __uint_as_float(raw.x & 0xffff0000u);
    out[2] = __uint_as_float(raw.y << 16);
    out[3] = __uint_as_float(raw.y & 0xffff0000u);
    out[4] = __uint_as_float(raw.z << 16);
    out[5] = __uint_as_float(raw.z & 0xffff0000u);
    out[6] = __uint_as_float(raw.w << 16);
    out[7] = __uint_as_float(raw.w & 0xffff0000u);
  }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// streaming read that is not expected to be reused soon
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- wave reductions
// Sum over the 64 lanes with DPP row operations (VALU, no LDS traffic); the
// total is read from lane 63 and returned to every lane.  The order of the
// additions is fixed, so the result is bit-identical run to run and in every
// workgroup that reduces the same values.
#define SPARK_DPP_ADD(v, ctrl, rmask)                                                                          \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rmask, 0xf, true))
__device__ __forceinline__ float wave_sum_dpp(float v) {
  SPARK_DPP_ADD(v, 0xb1, 0xf);   // quad_perm [1,0,3,2]
  SPARK_DPP_ADD(v, 0x4e, 0xf);   // quad_perm [2,3,0,1]
  SPARK_DPP_ADD(v, 0x114, 0xf);  // row_shr:4
  SPARK_DPP_ADD(v, 0x118, 0xf);  // row_shr:8   -> lane 15 of each row holds the row sum
  SPARK_DPP_ADD(v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  SPARK_DPP_ADD(v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3 -> lane 63 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
#undef SPARK_DPP_ADD

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (VALU only).
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
#define SPARK_DPP_SCAN(v, ctrl, rmask) v += __builtin_amdgcn_update_dpp(0, v, ctrl, rmask, 0xf, true)
  SPARK_DPP_SCAN(v, 0x111, 0xf);  // row_shr:1
  SPARK_DPP_SCAN(v, 0x112, 0xf);  // row_shr:2
  SPARK_DPP_SCAN(v, 0x114, 0xf);  // row_shr:4
  SPARK_DPP_SCAN(v, 0x118, 0xf);  // row_shr:8  -> prefix within each row of 16
  SPARK_DPP_SCAN(v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  SPARK_DPP_SCAN(v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef SPARK_DPP_SCAN
  return v;
}

// Set bits of the wave mask m that belong to lanes below this one.
__device__ __forceinline__ int mbcnt64(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Sum over each row of 16 lanes (DPP within rows); every lane of a row gets
// its row's total.
__device__ __forceinline__ float row16_sum(float v) {
#define SPARK_DPP_ROW(v, ctrl) \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true))
  SPARK_DPP_ROW(v, 0xb1);   // quad_perm [1,0,3,2]
  SPARK_DPP_ROW(v, 0x4e);   // quad_perm [2,3,0,1]
  SPARK_DPP_ROW(v, 0x124);  // row_ror:4
  SPARK_DPP_ROW(v, 0x128);  // row_ror:8
#undef SPARK_DPP_ROW
  return v;
}

// Column sums of NV per-lane values (NV a power of two, at most 64) over the
// 64 lanes of a wave, all columns at once: at each step a lane hands half of
// the values it still holds to its partner (lane xor m) and adds the other
// half to what it receives, so after log2(NV) steps every lane holds a
// partial of one column, col; the remaining steps add over the lanes that
// share a column.  Every lane returns the full sum of its column col.
template <int NV>
__device__ __forceinline__ float wave_colsum(float (&v)[NV], int lane, int& col) {
  constexpr int S = NV >= 64 ? 6 : NV >= 32 ? 5 : NV >= 16 ? 4 : NV >= 8 ? 3 : NV >= 4 ? 2 : NV >= 2 ? 1 : 0;
  static_assert((1 << S) == NV, "NV must be a power of two");
  col = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int m = 32 >> s, h = NV >> (s + 1);
    const uint32_t upm = (lane & m) ? 0xffffffffu : 0u;  // bit mask select: no selects of array slots
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + h]);
      const float give = __uint_as_float((a & upm) | (b & ~upm));
      const float keep = __uint_as_float((b & upm) | (a & ~upm));
      v[i] = keep + __shfl_xor(give, m, kWave);
    }
    col += (lane & m) ? h : 0;
  }
  float t = v[0];
#pragma unroll
  for (int m = 32 >> S; m >= 1; m >>= 1) t += __shfl_xor(t, m, kWave);
  return t;
}

// Butterfly reductions: every lane ends with the same value, bit for bit
// (each step adds a and b in either order, and fp add is commutative).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float bcast0(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

// Exclusive prefix sum of a per-lane int across the wave (lanes in order).
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x - v;
}

// (count, mean, M2) of a set of values, merged by Chan et al.'s pairwise rule.
struct Moments {
  float n, mean, m2;
};
__device__ __forceinline__ Moments merge(const Moments& a, const Moments& b) {
  const float n = a.n + b.n;
  if (n == 0.f) return a;
  const float d = b.mean - a.mean;
  const float fb = b.n / n;
  Moments r;
  r.n = n;
  r.mean = a.mean + d * fb;
  r.m2 = a.m2 + b.m2 + d * d * a.n * fb;
  return r;
}
// Merge the per-lane moments of a wave in a fixed butterfly order; the result
// is taken from lane 0 so that every lane (and every workgroup running the same
// code on the same data) holds identical bits.
__device__ __forceinline__ Moments wave_merge(Moments m) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    Moments o;
    o.n = __shfl_xor(m.n, s, kWave);
    o.mean = __shfl_xor(m.mean, s, kWave);
    o.m2 = __shfl_xor(m.m2, s, kWave);
    // the lower lane of each pair is always the left operand
    const bool low = (__lane_id() & s) == 0;
    m = low ? merge(m, o) : merge(o, m);
  }
  Moments r;
  r.n = bcast0(m.n);
  r.mean = bcast0(m.mean);
  r.m2 = bcast0(m.m2);
  return r;
}

// ---------------------------------------------------------------- activations
// GELU, tanh form: 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
// GELU, tanh form: 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3),
// evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)): one
// exponential and one division, and no cancellation for either sign of v.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float c2 = 1.5957691216057308f;  // 2 sqrt(2/pi)
  return v / (1.f + __expf(-c2 * (v + 0.044715f * v * v * v)));
}
// softplus log(1 + e^v) in the overflow-free form max(v,0) + log1p(e^-|v|).
__device__ __forceinline__ float softplus(float v) { return fmaxf(v, 0.f) + log1pf(__expf(-fabsf(v))); }

// The same on the hardware exp2/log2/reciprocal (v_exp_f32, v_log_f32,
// v_rcp_f32, about 1 ulp each): log1p(e) for e = e^-|v| in (0, 1] as
// log(u) * e / (u - 1) with u = 1 + e in [1, 2] (the rounding of u cancels in
// the ratio; u - 1 is exact), and e itself when u rounds to 1.
__device__ __forceinline__ float softplus_fast(float v) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(v));
  const float u = 1.f + e;
  const float l = u == 1.f ? e : (0.6931471805599453f * __builtin_amdgcn_logf(u)) * (e * __builtin_amdgcn_rcpf(u - 1.f));
  return fmaxf(v, 0.f) + l;
}

// ---------------------------------------------------------------- tagged words
// Cross-workgroup exchange inside one persistent kernel.  A published value is
// a 64-bit word {value bits, 32-bit tag} written and read with device-scope
// relaxed atomics, which are coherent across the XCDs' separate L2 caches.
// The reader accepts a word only when its tag equals the tag of the exchange
// it waits for, so no fence is needed between different words.
__device__ __forceinline__ void put_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_tagged_u32(uint64_t* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait (bounded) for the word at p to carry `tag`; returns its low 32 bits.
// On timeout sets *fail and returns 0.
__device__ __forceinline__ uint32_t wait_tagged(const uint64_t* p, uint32_t tag, uint32_t spin_limit, bool* fail) {
  uint64_t w = get_word(p);
  uint32_t spins = 0;
  while ((uint32_t)(w >> 32) != tag) {
    if (++spins > spin_limit || *fail) {
      *fail = true;
      return 0u;
    }
    w = get_word(p);
  }
  return (uint32_t)w;
}

__device__ __forceinline__ int xcc_id() {
  // HW_REG_XCC_ID: index of the XCD this wave runs on, bits [3:0]
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 7;
}

}  // namespace spark
