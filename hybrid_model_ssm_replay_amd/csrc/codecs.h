// Storage codecs of the split-precision state, device side.
//
// The read copy and the recurrence checkpoint may use different precisions,
// so that the read copy's rounding never re-enters the recurrence [P1,
// Interpretation 4; P3, Interpretation 3].  Formats (bit-exact definitions,
// identical to those the parity tests check against):
//   e4m3  OCP FP8 e4m3fn, round to nearest even, saturating at +-448, no
//         negative zero;
//   e2m1  4-bit {0, 0.5, 1, 1.5, 2, 3, 4, 6} x sign, one e4m3 scale per 16
//         consecutive elements: s = e4m3(amax / 6) (correctly rounded float32
//         division); element codes decided by exact comparisons of |x| with
//         the midpoints t s (t s is exact in float32); even element in the low
//         nibble; a zero magnitude carries no sign;
//   f16sr IEEE binary16 with stochastic rounding
//         SR(x, r) = RTZ16(x + sign(x) (r / 2^24) ulp16(|x|)), saturating at
//         +-65504, with r the top 24 bits of one Philox-4x32-10 output word.
// Decoding is exact and uses the gfx950 conversion instructions: fp8 through
// v_cvt_pk_f32_fp8 (OCP e4m3fn), fp4 through v_cvt_scalef32_pk_f32_fp4 at
// scale 1 (that instruction applies only the exponent of its scale operand, so
// the e4m3 block scale is multiplied in afterwards).  e4m3 encoding uses
// v_cvt_pk_fp8_f32 (round to nearest even) on values clamped to +-448, then
// clears the sign of zero codes; measured equal to the definition above on
// every e4m3 value and midpoint (and their float32 neighbours) and on 4M
// random values.  The element encoders are branch-free: a divergent branch
// per element costs more than the arithmetic.
#pragma once

#include <hip/hip_fp16.h>

#include "common.h"

namespace rssm {

// ---- Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ------------------------
struct Philox4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return Philox4{c0, c1, c2, c3};
}

// ---- e4m3 ------------------------------------------------------------------
// Four values into one word, value i in byte i.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.f, 448.f), cb = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  const float cc = __builtin_amdgcn_fmed3f(c, -448.f, 448.f), cd = __builtin_amdgcn_fmed3f(d, -448.f, 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, lo, true);
  // A byte whose low 7 bits are zero keeps no sign (no negative zero).
  const uint32_t nz = (w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;  // bit 7 of a byte: its low 7 bits are nonzero
  return w & (nz | 0x7F7F7F7Fu);
}

__device__ __forceinline__ uint32_t e4m3_encode(float x) { return e4m3_encode4(x, 0.f, 0.f, 0.f) & 0xFFu; }

__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFF, false);
  return v[0];
}

// ---- fp16 stochastic rounding ---------------------------------------------------
__device__ __forceinline__ float f16_sr(float x, uint32_t r24) {
  const float a = fabsf(x);
  // fp16 normal range: add the top 13 random bits below the fp16 mantissa and truncate.
  const float mag_n = __uint_as_float((__float_as_uint(a) + (r24 >> 11)) & ~0x1FFFu);
  // fp16 subnormal range: units of 2^-24.
  const float v = a * 16777216.f;  // exact
  const float n = floorf(v);
  const float thr = (float)(0x1000000u - r24) * 5.9604644775390625e-08f;  // (2^24 - r) 2^-24, exact
  const float mag_s = (n + ((v - n) >= thr ? 1.f : 0.f)) * 5.9604644775390625e-08f;
  const float mag = fminf(a >= 6.103515625e-05f ? mag_n : mag_s, 65504.f);  // 2^-14: the fp16 normal range
  return x < 0.f ? -mag : mag;  // -0 takes the positive zero
}

// ---- e2m1 (magnitude code of an element against the block scale s > 0) ----------
// The midpoints t s (t = 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; exact in float32)
// of one block; a tie goes to the even code, so the thresholds into odd codes
// are strict and those into even codes inclusive.
struct E2m1Thr {
  float t[7];
};

__device__ __forceinline__ E2m1Thr e2m1_thresholds(float s) {
  return E2m1Thr{{0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.f * s}};
}

// The code counts the midpoints below |x| (branch-free: a divergent branch per
// element costs more than the seven comparisons).
__device__ __forceinline__ uint32_t e2m1_code(float x, const E2m1Thr &th) {
  const float a = fabsf(x);
  const uint32_t m = (uint32_t)(a > th.t[0]) + (uint32_t)(a >= th.t[1]) + (uint32_t)(a > th.t[2]) +
                     (uint32_t)(a >= th.t[3]) + (uint32_t)(a > th.t[4]) + (uint32_t)(a >= th.t[5]) +
                     (uint32_t)(a > th.t[6]);
  return m | ((x < 0.f && m != 0) ? 8u : 0u);
}

// Two e2m1 values from byte `sel` (0..3) of `w`, low nibble first, unscaled.
template <int SEL>
__device__ __forceinline__ float2 e2m1_pair(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

}  // namespace rssm
