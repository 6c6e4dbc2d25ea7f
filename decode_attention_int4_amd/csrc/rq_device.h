// rq_device.h -- device-side number-format helpers for gfx950.
//
// FP8 here is OCP E4M3 "fn" (bias 7, 3 mantissa bits, subnormals m*2^-9, no
// infinities, max 448).  Encoding from double rounds to nearest with ties to
// even on the mantissa bits, saturates at +-448 and keeps the sign of zero.
// BF16 encoding from double rounds once, directly from the double's bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

// ---------------------------------------------------------------- decoding
__device__ __forceinline__ float fp8_to_f32(uint32_t b) {
  // Rebuild the value as an fp32 bit pattern: exponent bias 7 -> 127, the
  // 3 mantissa bits move to the top of the fp32 mantissa.  Subnormals
  // (exponent field 0) are m * 2^-9.
  const uint32_t s = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t m = b & 7u;
  float mag;
  if (e == 0)
    mag = (float)m * 0.001953125f;  // 2^-9
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | s);
}

__device__ __forceinline__ double fp8_to_f64(uint32_t b) { return (double)fp8_to_f32(b); }

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---------------------------------------------------------------- encoding
// Rounds x (a double) to FP8 e4m3fn, half to even, without branches: with e
// the exponent of |x| clamped below at -6 (the subnormal range shares the
// quantum 2^-9 of exponent -6), k = rint(|x| * 2^(3-e)) is the mantissa
// (8..16 for normals, 0..8 below) and the code is (e + 7) * 8 + k - 8; k = 16
// carries into the next exponent by that same formula.  |x| >= 448
// saturates to 0x7E, NaN gives 0x7F, the sign bit is x's.
__device__ __forceinline__ uint32_t f64_to_fp8(double x) {
  const uint32_t hi = (uint32_t)((uint64_t)__double_as_longlong(x) >> 32);
  const uint32_t sign = (hi >> 31) << 7;
  const double a = fabs(x);
  const int e = (int)((hi >> 20) & 0x7FFu) - 1023;
  const int eq = e > -6 ? e : -6;
  const double k = rint(ldexp(a, 3 - eq));
  uint32_t code = (uint32_t)(((eq + 7) << 3) + (int)k - 8);
  code = a >= 448.0 ? 0x7Eu : code;
  code = a != a ? 0x7Fu : code;
  return sign | code;
}

__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(bits >> 63) << 15;
  const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
  const double a = __longlong_as_double((long long)mag);
  if (a != a) return 0x7FC0u;
  if (mag == 0) return sign;
  const int e = (int)(mag >> 52) - 1023;
  if (e < -126) {
    // BF16 subnormals: k * 2^-133; k == 128 is the smallest normal (code 0x80).
    const double k = rint(a * 0x1p133);
    return sign | (uint32_t)k;
  }
  const uint64_t frac = mag & 0x000FFFFFFFFFFFFFull;
  uint32_t q = (uint32_t)(frac >> 45);                 // top 7 mantissa bits
  const uint64_t rest = frac & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rest > half || (rest == half && (q & 1u))) ++q;
  int E = e;
  if (q == 128u) {
    q = 0;
    ++E;
  }
  if (E > 127) return sign | 0x7F80u;
  return sign | ((uint32_t)(E + 127) << 7) | q;
}

// fp32 -> BF16, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace rq
