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

// Lane exchange in registers.  The wave reductions and scans below use fixed lane patterns,
// which DPP (quad permutes, shifts and rotations inside 16-lane rows, row broadcasts) and
// v_permlane16/32_swap provide as VALU operations; a general shuffle (ds_bpermute) makes an
// LDS round trip for every step instead.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]: lane i takes lane i ^ 1
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]: lane i takes lane i ^ 2
constexpr int kRowShl = 0x100;      // + n: lane i of a 16-lane row takes lane i + n of the row
constexpr int kRowShr = 0x110;      // + n: lane i of a row takes lane i - n of the row
constexpr int kRowRor8 = 0x128;     // rotation by half a row: lane i takes lane i ^ 8
constexpr int kWaveShr1 = 0x138;    // lane i takes lane i - 1 of the wave (lane 0: none)
constexpr int kRowBcast15 = 0x142;  // row r takes lane 15 of row r - 1 (rows 1..3)
constexpr int kRowBcast31 = 0x143;  // rows 2 and 3 take lane 31
}  // namespace dpp

// The value x holds in lane (lane ^ O), for O a power of two below 64.  Every lane of the
// wave must be active.
template <int O>
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "xor distance");
  const int xi = (int)x;
  if constexpr (O == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, dpp::kQuadXor1, 0xF, 0xF, false);
  } else if constexpr (O == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, dpp::kQuadXor2, 0xF, 0xF, false);
  } else if constexpr (O == 4) {
    // lanes with bit 2 clear read four lanes up their row, the others four lanes down
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, xi, dpp::kRowShl + 4, 0xF, 0xF, false);
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, xi, dpp::kRowShr + 4, 0xF, 0xF, false);
    return (__lane_id() & 4) ? dn : up;
  } else if constexpr (O == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, dpp::kRowRor8, 0xF, 0xF, false);
  } else if constexpr (O == 16) {
    // swapping the odd rows of one copy with the even rows of another leaves rows (0,0,2,2)
    // in the first and (1,1,3,3) in the second
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    // likewise by halves: (low, low) in the first, (high, high) in the second
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}

// The value x holds in lane (lane - 1); 0 in lane 0.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t lane_before(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, dpp::kWaveShr1, 0xF, 0xF, false);
}

template <int O, typename T>
__device__ __forceinline__ T lane_xor(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lane values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, lane_xor32<O>(__builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xor32<O>((uint32_t)u);
    const uint64_t hi = lane_xor32<O>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, (hi << 32) | lo);
  }
}

// v = op(v, v of lane ^ O) for O = 32, 16, ..., 1: every lane ends with the reduction of the
// wave (for a commutative op the same value in every lane).
template <typename T, typename Op>
__device__ __forceinline__ T wave_butterfly(T v, Op op) {
  v = op(v, lane_xor<32>(v));
  v = op(v, lane_xor<16>(v));
  v = op(v, lane_xor<8>(v));
  v = op(v, lane_xor<4>(v));
  v = op(v, lane_xor<2>(v));
  v = op(v, lane_xor<1>(v));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_butterfly(v, [](T a, T b) { return a + b; });
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_butterfly(v, [](T a, T b) { return max(a, b); });
}

// inclusive prefix sum across the 64 lanes of a wave (exact: integer adds): the sum inside
// each 16-lane row by shifts of 1, 2, 4 and 8 lanes (lanes before the row start add 0),
// then the totals of the earlier rows through the row broadcasts
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowShr + 1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowShr + 2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowShr + 4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowShr + 8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kRowBcast31, 0xC, 0xF, false);
  return v;
}

// inclusive prefix maximum across the 64 lanes of a wave, for values below 2^31 (the same
// steps as the prefix sum)
__device__ __forceinline__ uint32_t wave_inclusive_max_scan(uint32_t v) {
  int x = (int)v;
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowShr + 1, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowShr + 2, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowShr + 4, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowShr + 8, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowBcast15, 0xA, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, dpp::kRowBcast31, 0xC, 0xF, false));
  return (uint32_t)x;
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
