// GELU in fp32 from IEEE-exact operations only, shared by the GPU kernels and
// the host program that tabulates it (gen_gelu_table.cpp).
//
// "Qwen-Image-2.1: TE AutoRound-AWQ on GPU + all-resident single-3090
// stack", section "Whole-pipeline follow-up": the int8 DiT path fuses the
// activation with the quantisation of the next linear's input. The
// activation of a DiT FFN is GELU, z Phi(z) (erf form), or its tanh form
// 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
//
// Every step is an IEEE operation with one rounding: fp32 add, multiply,
// fused multiply-add, correctly rounded division, and integer bit moves.
// Compiled without contraction (hipcc and the host compiler both take
// -ffp-contract=off; the GPU build also takes correctly rounded division),
// the host and the device therefore compute the same bits for every input,
// subnormal results included (fp32 denormals are kept on both). That is
// what lets the whole bf16 -> bf16 map be tabulated on the host at build
// time and looked up on the GPU.
//
//   erf form:  (0.5 z) erfc(-z / sqrt 2), with erfc(x) = t exp(-x^2 + P(t)),
//              t = 1 / (1 + x/2), x = |z| / sqrt 2, and 2 - erfc(x) for z > 0
//              (the form of the Chebyshev erfc of Numerical Recipes, section
//              6.2; P is our own degree-9 fit, erfc_poly.h).
//   tanh form: with t = sqrt(2/pi) (z + 0.044715 z^3) and e = exp(-2|t|),
//              z / (1 + e) for t >= 0 and z e / (1 + e) for t < 0 (the same
//              function as 0.5 z (1 + tanh t), without the overflow of
//              exp(-2t) for t << 0).
//   exp:       2^q by range reduction, q = n + f with n = rint(q), |f| <= 1/2,
//              2^f by its Taylor polynomial in f ln 2 to degree 7 (truncation
//              below 0.1 fp32 ulp; about 1.2 ulp with the rounding of the
//              Horner steps), scaled by 2^n built from its exponent bits.
//              Where q < -64 the evaluation takes 2^(q + 64) and scales the
//              result back by 2^-64 at the end, so that results in the
//              subnormal range are kept; below q = -190.5 every result is
//              below half the smallest subnormal, and 2^q is taken as 0.
#pragma once

#include <stdint.h>

#include "erfc_poly.h"

#if defined(__HIPCC__)
#define W8A8_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define W8A8_HD inline
#endif

namespace w8a8 {
namespace gelu {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kRsqrt2 = 0.707106781186547524f;         // 1 / sqrt 2
constexpr float kSqrt2OverPi = 0.797884560802865355f;    // sqrt(2 / pi)

// (ln 2)^k / k!, k = 0..7
constexpr float kExp2Poly[8] = {
    0x1.0000000000000p+0f,  0x1.62e4300000000p-1f, 0x1.ebfbe00000000p-3f, 0x1.c6b08e0000000p-5f,
    0x1.3b2ab60000000p-7f,  0x1.5d87fe0000000p-10f, 0x1.4309120000000p-13f, 0x1.ffcbfc0000000p-17f,
};

W8A8_HD float fma32(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// 2^q for q <= 127; 0 below q = -126.5 (and for a NaN q).
W8A8_HD float exp2_f32(float q) {
  if (!(q >= -126.5f)) return 0.0f;
  if (q > 127.0f) return __builtin_bit_cast(float, 0x7f800000u);
  const float n = (q + 0x1.8p23f) - 0x1.8p23f;      // rint(q), half to even (|q| < 2^22)
  const float f = q - n;                              // exact, |f| <= 1/2
  float p = kExp2Poly[7];
  for (int k = 6; k >= 0; --k) p = fma32(p, f, kExp2Poly[k]);
  const uint32_t e = (uint32_t)((int)n + 127) << 23;  // 2^n, -126 <= n <= 127
  return p * __builtin_bit_cast(float, e);
}

W8A8_HD float gelu_erf(float z) {
  const float x = __builtin_fabsf(z) * kRsqrt2;
  const float t = 1.0f / fma32(x, 0.5f, 1.0f);
  float p = kErfcPoly[kErfcPolyDegree];
  for (int i = kErfcPolyDegree - 1; i >= 0; --i) p = fma32(p, t, kErfcPoly[i]);
  const float q = (p - x * x) * kLog2e;
  const bool shifted = q < -64.0f;
  const float c = t * exp2_f32(shifted ? q + 64.0f : q);   // erfc(x) (* 2^64)
  const bool pos = z > 0.0f;
  const float y = (0.5f * z) * (pos ? 2.0f - (shifted ? 0.0f : c) : c);   // erfc(-x) = 2 - erfc(x)
  return (shifted && !pos) ? y * 0x1p-64f : y;
}

W8A8_HD float gelu_tanh(float z) {
  const float z3 = (z * z) * z;
  const float t = kSqrt2OverPi * (z + 0.044715f * z3);
  const float q = (-2.0f * kLog2e) * __builtin_fabsf(t);
  const bool shifted = q < -64.0f;
  const float e = exp2_f32(shifted ? q + 64.0f : q);       // exp(-2|t|) (* 2^64)
  const float r = 1.0f / (1.0f + (shifted ? 0.0f : e));
  const bool pos = t >= 0.0f;
  const float y = (pos ? z : z * e) * r;
  return (shifted && !pos) ? y * 0x1p-64f : y;
}

// fp32 -> bf16 bits, round to nearest even (finite and infinite values; a
// NaN becomes a quiet NaN).
W8A8_HD uint32_t to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace gelu
}  // namespace w8a8
