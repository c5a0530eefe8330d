// Element conversions with explicit rounding (round to nearest, ties to even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two packed bfloat16 / float16 (element 0 in the low half), one
// v_cvt_pk_{bf16,f16}_f32 each (round to nearest even).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2(f, 0.0f) & 0xffffu);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 x;
  __builtin_memcpy(&x, &h, 2);
  return static_cast<float>(x);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 x = static_cast<_Float16>(f);  // v_cvt_f16_f32: round to nearest even
  uint16_t h;
  __builtin_memcpy(&h, &x, 2);
  return h;
}

// float64 -> bfloat16 with a single rounding to nearest even, without
// branches.  From magnitude 2^-126 up, x is rounded to binary32 by
// round-to-odd (the hardware's nearest-even result, stepped one unit toward
// zero if it went away from zero, with its last bit set whenever the
// conversion was inexact), which keeps 16 bits below bfloat16's last place,
// so rounding that value to nearest even (v_cvt_pk_bf16_f32) gives the same
// result as rounding x itself; NaN stays NaN and infinities stay infinite.
// Below 2^-126 bfloat16 has the fixed quantum 2^-133: x is rounded to a
// multiple of it in binary64 (exact) and converted exactly.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const double ax = fabs(x);
  const float f = static_cast<float>(x);
  const double back = static_cast<double>(f);
  const bool inexact = back != x;
  uint32_t u = __float_as_uint(f);
  u -= (inexact && fabs(back) > ax) ? 1u : 0u;
  u |= inexact ? 1u : 0u;
  const float tiny = static_cast<float>(rint(x * 0x1p133) * 0x1p-133);
  return f32_to_bf16(ax < 0x1p-126 ? tiny : __uint_as_float(u));
}

// Storage dtype helpers for user buffers (0 = f32, 1 = bf16, 2 = f16).
__device__ __forceinline__ float load_as_f32(const void* p, int64_t idx, int dtype) {
  if (dtype == 0) return static_cast<const float*>(p)[idx];
  uint16_t h = static_cast<const uint16_t*>(p)[idx];
  return dtype == 1 ? bf16_to_f32(h) : f16_to_f32(h);
}

__device__ __forceinline__ void store_from_f32(void* p, int64_t idx, int dtype, float v) {
  if (dtype == 0) {
    static_cast<float*>(p)[idx] = v;
  } else {
    static_cast<uint16_t*>(p)[idx] = dtype == 1 ? f32_to_bf16(v) : f32_to_f16(v);
  }
}

// Operand types: OP = 0 f32, 1 bf16, 2 f16.
template <int OP> struct OpT;
template <> struct OpT<0> {
  using T = float;
  static __device__ __forceinline__ float to_f(T x) { return x; }
  static __device__ __forceinline__ T from_f(float x) { return x; }
};
template <> struct OpT<1> {
  using T = uint16_t;
  static __device__ __forceinline__ float to_f(T x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ T from_f(float x) { return f32_to_bf16(x); }
};
template <> struct OpT<2> {
  using T = uint16_t;
  static __device__ __forceinline__ float to_f(T x) { return f16_to_f32(x); }
  static __device__ __forceinline__ T from_f(float x) { return f32_to_f16(x); }
};

// Element index of (r, k) in an operand buffer with row length K.  16-bit
// operands: packed fragment layout, blocks of 32 rows x 64 k (4 KB) ordered by
// (row block, k block); inside, four 1 KB MFMA fragments (k-steps of 16), each
// holding lane l = 32 * ((k % 16) / 8) + r % 32 with 8 consecutive k.  fp32
// (check path): row-major.
template <int OP>
__device__ __forceinline__ int64_t op_index(int r, int k, int K) {
  if constexpr (OP == 0) {
    return static_cast<int64_t>(r) * K + k;
  } else {
    return ((static_cast<int64_t>(r >> 5) * (K >> 6) + (k >> 6)) << 11) + (((k >> 4) & 3) << 9) +
           (((((k >> 3) & 1) << 5) | (r & 31)) << 3) + (k & 7);
  }
}

}  // namespace muon
