// Device helpers shared by the gfx950 kernels of libw8a8.
//
// Numerics (the per-row symmetric int8 quantisation and the fp32 scale
// epilogue of the W8A8 int8-dynamic linear; Issue 5 probe, "Round two"):
//   scale = fl32(amax / 127); q = clamp(rint(fl32(x / scale)), -127, 127)
//   y = bf16_rne(((fl32(acc) * s_a) * s_w) + bias)
// The same maths serves fp16 activations/weights/bias/output (the guide
// quantises bf16 and fp16 weights): every helper that reads or writes 16-bit values takes
// the type as a template flag (F16 = false: bf16).
// Everything here is compiled with -ffp-contract=off so that no product and
// sum are fused, and with IEEE (correctly rounded) fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// An offset past every buffer descriptor bound: a load there reads zero, a
// store there is dropped (used to mask lanes without branches).
constexpr uint32_t kOOB = 0x7ffffff0u;

// Raw buffer descriptor over `bytes` bytes from `base` (bounds-checked,
// 32-bit offsets; loads past the bound return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte buffer load.
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// 16-byte non-temporal buffer load (nt), for data read exactly once.
__device__ __forceinline__ uint4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// still in flight (expcnt, lgkmcnt: no wait). gfx9 encoding: vmcnt[3:0] in
// bits 3:0 and vmcnt[5:4] in bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier on LDS traffic only (lgkmcnt 0, no fence): this wave's
// outstanding global loads and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0); vmcnt and expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp16 bits -> fp32 (exact; fp16 subnormals are kept: the f16 denormal mode
// of these kernels is IEEE).
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <bool F16>
__device__ __forceinline__ float half_to_f32(uint32_t bits16) {
  if constexpr (F16) return f16_to_f32(bits16);
  else return bf16_to_f32(bits16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> fp16 bits by the hardware conversion (round to nearest even in the
// default mode, subnormal results kept, overflow to infinity).
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <bool F16>
__device__ __forceinline__ uint32_t f32_to_half_rne(float f) {
  if constexpr (F16) return f32_to_f16_rne(f);
  else return f32_to_bf16_rne(f);
}

// Per-row scale from the largest |x| bit pattern (bf16 and fp16 magnitudes
// both compare as integers). One IEEE division.
template <bool F16 = false>
__device__ __forceinline__ float row_scale(uint32_t amax_bits16) {
  return half_to_f32<F16>(amax_bits16) / 127.0f;
}

// Quantisation of one value: round(fl32(x / s)) half to even, clamped to
// [-127, 127], computed as rint(P) for the exact product P = x * r, with
// r = fl32(1 / s) for a normal s. P is never rounded on its own: it enters
// one fma, m = fl32(P + 1.5 * 2^23).
//
// r = (1/s)(1 + d) with |d| <= u (u = 2^-24), so P differs from the exact
// quotient Q = x/s by at most |Q|u, and fl32(Q) differs from Q by at most
// |Q|u. |Q| <= amax/s <= 127 / (1 - u), so |P - fl32(Q)| < 254.01u < 2^-16.
// Every value in [2^23, 2^24) is an integer, so m = 1.5 * 2^23 + rint(P)
// (round to nearest even), rint(P) = m - 1.5 * 2^23 exactly, and the low
// byte of m's bit pattern is rint(P) as a two's-complement int8 (|P| <
// 127.5, so no clamp). The distance e = fl32(P - rint(P)) is a second fma
// (|P - rint(P)| <= 1/2, so it rounds by at most 2^-26). If |e| <
// 1/2 - 2^-15, then |fl32(Q) - rint(P)| < 1/2 - 2^-15 + 2^-26 + 2^-16 <
// 1/2 and rint(fl32(Q)) == rint(P). Otherwise the value lies near a
// rounding boundary and the caller redoes it with the IEEE division.
// Returns m's bits; dist receives |e|.
constexpr float kRoundMagic = 12582912.0f;   // 1.5 * 2^23
constexpr float kNearHalf = 0.5f - 0x1p-15f;

__device__ __forceinline__ uint32_t quant_fma(float x, float r, float& dist) {
  const float m = __builtin_fmaf(x, r, kRoundMagic);
  // kRoundMagic - m is -rint(P), exactly
  dist = __builtin_fabsf(__builtin_fmaf(x, r, kRoundMagic - m));
  return __float_as_uint(m);
}

// Exact route: one IEEE division, rounded half to even and clamped (a
// subnormal scale can carry the quotient past 127.5). Used near rounding
// boundaries and for rows whose scale is subnormal (1/s would overflow or
// lose precision). Returns the int8 in the low byte.
__device__ __forceinline__ uint32_t quant_div(float x, float s) {
  return (uint32_t)(int)__builtin_amdgcn_fmed3f(__builtin_rintf(x / s), -127.0f, 127.0f);
}

// Low bytes of four words, packed little-endian (a in byte 0).
__device__ __forceinline__ uint32_t pack_low_bytes4(uint32_t a, uint32_t b, uint32_t c,
                                                    uint32_t d) {
  // v_perm_b32: selector bytes 0-3 pick from the second operand, 4-7 from
  // the first, 12 gives zero
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Quantises eight bf16 (or fp16) values (one 16-byte load) with scale s
// (r = 1/s) into eight int8 packed little-endian in a uint2. A zero scale
// (all-zero row) gives zeros. The division fallback is taken for the whole
// chunk, once per wave, only when some lane has a value near a rounding
// boundary (or the scale is subnormal), so the common path has no
// per-element branch.
template <bool F16 = false>
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float r, bool zero, bool exact_div) {
  if (zero) return make_uint2(0u, 0u);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = half_to_f32<F16>(w[i] & 0xffffu);
    x[2 * i + 1] = half_to_f32<F16>(w[i] >> 16);
  }
  // the largest distance of the eight decides whether any is near
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float d;
    q[i] = quant_fma(x[i], r, d);
    dmax = __builtin_fmaxf(dmax, d);
  }
  if (__builtin_amdgcn_ballot_w64(dmax >= kNearHalf || exact_div)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float d;
      quant_fma(x[i], r, d);
      if (d >= kNearHalf || exact_div) q[i] = quant_div(x[i], s);
    }
  }
  return make_uint2(pack_low_bytes4(q[0], q[1], q[2], q[3]), pack_low_bytes4(q[4], q[5], q[6], q[7]));
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

// Unsigned max over the 64 lanes of the wave (DPP within rows of 16, then
// row broadcasts), returned as a wave-uniform value. Every lane must be
// active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false)); // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false)); // row_ror 8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast 15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false)); // row_bcast 31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The weight scale and bias (converted to fp32) of output row
// n_base + (lane & 7) of a small-M wave, read through descriptors bounded at
// the wave's rows_valid rows (zero past them). The small-M kernels request
// these first: requested after the weight stream, they would be served last
// and hold the epilogue back. One pair per lane keeps two registers live
// across the stream; gather4 hands each epilogue lane the four it needs.
template <bool HAS_BIAS, bool F16>
__device__ __forceinline__ void load_row_scale(const float* w_scale, const uint16_t* bias,
                                               int64_t n_base, int rows_valid, int lane,
                                               float& sw, float& bb) {
  const uint32_t nv = rows_valid > 0 ? (uint32_t)rows_valid : 0u;
  const int64_t nb = rows_valid > 0 ? n_base : 0;
  const __amdgpu_buffer_rsrc_t r_sw = make_rsrc(w_scale + nb, nv * 4u);
  sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sw, (lane & 7) * 4, 0, 0));
  bb = 0.f;
  if constexpr (HAS_BIAS) {
    const __amdgpu_buffer_rsrc_t r_b = make_rsrc(bias + nb, nv * 2u);
    bb = half_to_f32<F16>(__builtin_amdgcn_raw_buffer_load_b16(r_b, (lane & 7) * 2, 0, 0));
  }
}

// out[r] = v of lane first + r (r = 0..3); every lane of the wave must be
// active.
__device__ __forceinline__ void gather4(float v, int first, float (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    out[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((first + r) * 4, __float_as_int(v)));
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
