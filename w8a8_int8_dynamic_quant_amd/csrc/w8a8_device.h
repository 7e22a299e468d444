// Device helpers shared by the gfx950 kernels of libw8a8.
//
// Numerics (the per-row symmetric int8 quantisation and the fp32 scale
// epilogue of the W8A8 int8-dynamic linear; Issue 5 probe, "Round two"):
//   scale = fl32(amax / 127); q = clamp(rint(fl32(x / scale)), -127, 127)
//   y = bf16_rne(((fl32(acc) * s_a) * s_w) + bias)
// Everything here is compiled with -ffp-contract=off so that no product and
// sum are fused, and with IEEE (correctly rounded) fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Per-row scale from the largest |x| bit pattern (bf16 magnitudes compare
// as integers). One IEEE division.
__device__ __forceinline__ float row_scale(uint32_t amax_bits16) {
  return bf16_to_f32(amax_bits16) / 127.0f;
}

// Rounds fl32(x / s) half to even and clamps to [-127, 127], where
// r = fl32(1 / s) and s is a normal fp32 number.
//
// t = fl32(x * r) differs from the exact quotient Q = x/s by at most
// |Q|(2u + u^2) and fl32(Q) differs from Q by at most |Q|u (u = 2^-24).
// |Q| <= amax/s <= 127 / (1 - u), so |t - fl32(Q)| < 2.3e-5 < 2^-15. If t is
// farther than 2^-15 from every half-integer, no rounding boundary lies
// between t and fl32(Q) and rint(t) == rint(fl32(Q)). Otherwise the exact
// division is taken. (t - rint(t) is exact by Sterbenz's lemma.)
__device__ __forceinline__ int quant_fast(float x, float s, float r) {
  float t = x * r;
  float rt = __builtin_rintf(t);
  float d = __builtin_fabsf(t - rt);
  if (__builtin_fabsf(0.5f - d) <= 0x1p-15f) rt = __builtin_rintf(x / s);
  rt = __builtin_fminf(__builtin_fmaxf(rt, -127.0f), 127.0f);
  return (int)rt;
}

// Exact route for every element: one IEEE division per element. Used for
// rows whose scale is subnormal (1/s would overflow or lose precision).
__device__ __forceinline__ int quant_div(float x, float s) {
  float rt = __builtin_rintf(x / s);
  rt = __builtin_fminf(__builtin_fmaxf(rt, -127.0f), 127.0f);
  return (int)rt;
}

// Quantises one bf16 value given the row's scale s and r = 1/s. A zero scale
// (all-zero row) gives 0; subnormal scales take the division route.
__device__ __forceinline__ int quant_one(uint32_t bits16, float s, float r, bool exact_div) {
  float x = bf16_to_f32(bits16);
  if (exact_div) return quant_div(x, s);
  return quant_fast(x, s, r);
}

// Quantises eight bf16 values (one 16-byte load) into eight int8 values
// packed little-endian in a uint2.
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float r, bool zero, bool exact_div) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
  if (!zero) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int lo = quant_one(w[i] & 0xffffu, s, r, exact_div);
      int hi = quant_one(w[i] >> 16, s, r, exact_div);
      uint32_t pair = (uint32_t)(lo & 0xff) | ((uint32_t)(hi & 0xff) << 8);
      out[i >> 1] |= pair << ((i & 1) * 16);
    }
  }
  return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ uint32_t absmax_bits8(uint4 v, uint32_t m) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7fffu);
    m = max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Scale epilogue for one element (fixed order, no contraction). Without a
// bias nothing is added, so a product that underflows to -0 stays -0.
template <bool HAS_BIAS>
__device__ __forceinline__ float epilogue_f32(int acc, float sa, float sw, float b) {
#pragma clang fp contract(off)
  float t = (float)acc;
  t = t * sa;
  t = t * sw;
  if (HAS_BIAS) t = t + b;
  return t;
}

}  // namespace w8a8
