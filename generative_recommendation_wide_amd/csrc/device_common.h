// Device helpers for gfx950 (wave64): number formats, ordered keys, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two OCP E4M3 ("fn") codes -> two floats, exact (hardware conversion; HI selects bytes
// 2..3 of the word instead of 0..1).
template <bool HI>
__device__ __forceinline__ floatx2 fp8x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
}

// A float that is exactly representable in bf16 (every E4M3 value is) -> its bf16 bits.
__device__ __forceinline__ uint32_t f32_exact_to_bf16_bits(float f) {
  return __float_as_uint(f) >> 16;
}

// Four E4M3 codes (one 32-bit word) -> four bf16 values packed in two 32-bit words, exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t word) {
  floatx2 lo = fp8x2_to_f32<false>(word);
  floatx2 hi = fp8x2_to_f32<true>(word);
  u32x2 r;
  r.x = f32_exact_to_bf16_bits(lo.x) | (f32_exact_to_bf16_bits(lo.y) << 16);
  r.y = f32_exact_to_bf16_bits(hi.x) | (f32_exact_to_bf16_bits(hi.y) << 16);
  return r;
}

// Order-preserving map of a float32 to uint32 (larger float -> larger key); -0.0 and +0.0
// map to the same key.  NaN never reaches it (callers filter NaN first).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose ordered key is k (for k = 0x7FFFFFFF, which no float maps to: -0.0).
__device__ __forceinline__ float float_of_ordered(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Composite selection key: ordered score key in the high word, ~flat in the low word, so
// that a larger composite means (key descending, flat ascending).
__device__ __forceinline__ uint64_t composite_key(uint32_t okey, uint32_t flat) {
  return ((uint64_t)okey << 32) | (uint64_t)(~flat);
}
__device__ __forceinline__ uint32_t composite_flat(uint64_t c) { return ~(uint32_t)c; }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// inclusive prefix sum across the 64 lanes of a wave
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Maximum that propagates NaN (IEEE 754-2019 maximum).  Chains of it lower to
// v_maximum3_f32; fmaxf on MFMA results costs an extra canonicalising v_max per operand.
// max(x[l], x[l ^ 32]) in every lane l: the two 32-lane halves exchanged in registers
// (v_permlane32_swap of x with itself leaves x[l] and x[l ^ 32] in the pair), with no LDS
// round trip as a cross-half shuffle takes.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace grw
