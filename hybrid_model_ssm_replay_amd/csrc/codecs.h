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
// the e4m3 block scale is multiplied in afterwards).
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
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const float a = fabsf(x);
  const uint32_t bits = __float_as_uint(a);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7E;
  } else if (a >= 0.015625f) {  // 2^-6: normal e4m3
    int e = (int)(bits >> 23) - 127;
    uint32_t r = (bits >> 20) & 7;
    const uint32_t rem = bits & 0xFFFFF;
    r += (rem > 0x80000u) || (rem == 0x80000u && (r & 1));
    if (r == 8) {
      r = 0;
      ++e;
    }
    code = (uint32_t)((e + 7) << 3) | r;
    code = code > 0x7E ? 0x7E : code;
  } else {
    code = (uint32_t)rintf(a * 512.f);  // steps of 2^-9, ties to even; exact scaling
  }
  return code | ((x < 0.f && code != 0) ? 0x80u : 0u);
}

__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFF, false);
  return v[0];
}

// ---- fp16 stochastic rounding ---------------------------------------------------
__device__ __forceinline__ float f16_sr(float x, uint32_t r24) {
  const float a = fabsf(x);
  float mag;
  if (a >= 6.103515625e-05f) {  // 2^-14: fp16 normal range
    const uint32_t t = (__float_as_uint(a) + (r24 >> 11)) & ~0x1FFFu;
    mag = __uint_as_float(t);
  } else {  // fp16 subnormal range: units of 2^-24
    const float v = a * 16777216.f;  // exact
    const float n = floorf(v);
    const float f = v - n;
    const float thr = (float)(0x1000000u - r24) * 5.9604644775390625e-08f;  // (2^24 - r) 2^-24, exact
    mag = (n + (f >= thr ? 1.f : 0.f)) * 5.9604644775390625e-08f;
  }
  mag = fminf(mag, 65504.f);
  return x < 0.f ? -mag : mag;
}

// ---- e2m1 (magnitude code of an element against the block scale s > 0) ----------
__device__ __forceinline__ uint32_t e2m1_code(float x, float s) {
  const float a = fabsf(x);
  uint32_t m;
  if (a <= 0.25f * s) m = 0;
  else if (a < 0.75f * s) m = 1;
  else if (a <= 1.25f * s) m = 2;
  else if (a < 1.75f * s) m = 3;
  else if (a <= 2.5f * s) m = 4;
  else if (a < 3.5f * s) m = 5;
  else if (a <= 5.f * s) m = 6;
  else m = 7;
  return m | ((x < 0.f && m != 0) ? 8u : 0u);
}

// Two e2m1 values from byte `sel` (0..3) of `w`, low nibble first, unscaled.
template <int SEL>
__device__ __forceinline__ float2 e2m1_pair(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

}  // namespace rssm
