// Producers fused with the per-row int8 activation quantisation (gfx950).
//
// "Qwen-Image-2.1: TE AutoRound-AWQ on GPU + all-resident single-3090
// stack", section "Whole-pipeline follow-up": around its int8 GEMMs the W8A8
// DiT path runs fused activation-quantisation, normalisation and activation
// kernels. Here the normalisation is the modulated LayerNorm of a DiT block,
//   y = bf16((x - mean) / sqrt(var + eps) * (1 + scale) + shift)
// (mean and biased variance over the row; shift and scale are bf16 [K] per
// group of rows), and the activation is GELU, y = bf16(z Phi(z)), or its tanh
// form. Each kernel writes the int8 codes and the fp32 scale of y, quantised
// exactly as the activation quantisation does (scale = amax / 127, round half
// to even), and, when asked, y itself: what the unfused producer would have
// written and the quantisation would have read back.
//
// Layout and schedule follow the quantisation kernels: one, two or four
// waves per row (two from K > 1024, four from K > 4096), lane `lane` of wave part p
// holding the row's 16-byte chunks lane + 64 (p + WPR c), c < CH, all
// requested at once (non-temporal: x is read once) and kept in registers
// through every step, so the row is read from HBM once and written once as
// int8. Chunks past K read zero through the bounded buffer descriptor and are
// masked out of the sums and the amax.
//
// fp32 evaluation (no contraction; correctly rounded division and square
// root):
//   LayerNorm: each lane sums its 8 CH values in order, a 64-lane butterfly
//   adds the lanes (every lane ends with the same value) and the WPR wave
//   sums are added in part order: no term passes through more than
//   K / 64 + 16 additions. mean = sum / K, var = (sum of (x - mean)^2) / K
//   (squares accumulated by fused multiply-add), rstd = 1 / sqrt(var + eps),
//   y = fma(fma(x, rstd, -(mean rstd)), 1 + scale, shift): two roundings
//   fewer than the literal order, and the rounding of mean rstd is within
//   the error the mean itself carries (u |mean| rstd).
//   GELU: (0.5 z) * erfc(-z / sqrt 2), which has no cancellation for z << 0,
//   with erfc(x) = t exp(-x^2 + P(t)), t = 1 / (1 + x/2), for x = |z| / sqrt 2
//   (2 - erfc(x) for z > 0): the form of Numerical Recipes' Chebyshev erfc
//   (section 6.2), P a degree-9 polynomial of our own fit, within 2 fp32 ulps
//   (gen_erfc_poly.py).
//   tanh form: with t = sqrt(2/pi) (z + 0.044715 z^3) and e = exp(-2|t|),
//   z / (1 + e) for t >= 0 and z e / (1 + e) for t < 0 (the same function as
//   0.5 z (1 + tanh t), without the overflow of exp(-2t) at t << 0).
//   exp and 1/x are the hardware's v_exp_f32 (2^x) and v_rcp_f32 (each within
//   about an ulp); an exponent below -64 is raised by 64 and the result scaled
//   back by 2^-64 at the end, so that results in the subnormal range are kept.
//   The bf16 rounding is v_cvt_pk_bf16_f32 (nearest even, subnormals kept).
//
// GELU on large inputs goes through a table instead: a bf16 input has 65536
// values, so the whole map z -> bf16(GELU(z)) is 128 KB, which fits in one
// compute unit's 160 KB of LDS. A small kernel evaluates the map with the
// fp32 code above (the same bits the per-element kernel produces) into a
// static device array on the caller's stream; the quantisation kernel then
// copies it into LDS once per workgroup (one 1024-thread workgroup per
// compute unit, four rows at a time, four waves to a row) and replaces the ~30 VALU
// instructions per element of the formula by one LDS lookup, leaving the row
// stream HBM-bound. Every call rebuilds the table with the same values, so
// calls on different streams only ever write identical bytes.
#include "erfc_poly.h"
#include "producers.h"
#include "row_groups.h"
#include "w8a8_device.h"

namespace w8a8 {

namespace {

__device__ __forceinline__ void store8(uint2 q, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64((v2u){q.x, q.y}, r, off, 0, 0);
}

__device__ __forceinline__ void store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128((v4u){v.x, v.y, v.z, v.w}, r, off, 0, 0);
}

// Sum over the 64 lanes by a butterfly: at each step lanes i and i ^ off add
// the same two values, so every lane ends with the same sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Eight fp32 -> eight bf16 (round to nearest even), packed low to high.
__device__ __forceinline__ uint4 pack8_bf16(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){f[2 * i], f[2 * i + 1]}, v2bf));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr float kLog2e = 1.44269504088896341f;

// GELU in fp32 without branches. 2^q comes from v_exp_f32; where q < -64 it
// is taken as 2^(q + 64) and the result scaled back by 2^-64 at the end, so
// results in the fp32 subnormal range are kept. On the positive side such a
// term is below 2^-64 and drops out of 1 + e (or 2 - erfc) exactly.
__device__ __forceinline__ float gelu_erf(float z) {
#pragma clang fp contract(off)
  const float x = __builtin_fabsf(z) * 0.707106781186547524f;     // |z| / sqrt 2
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(x, 0.5f, 1.0f));
  float p = kErfcPoly[kErfcPolyDegree];
#pragma unroll
  for (int i = kErfcPolyDegree - 1; i >= 0; --i) p = __builtin_fmaf(p, t, kErfcPoly[i]);
  const float q = (p - x * x) * kLog2e;
  const bool shifted = q < -64.0f;
  const float c = t * __builtin_amdgcn_exp2f(shifted ? q + 64.0f : q);   // erfc(x) (* 2^64)
  const bool pos = z > 0.0f;
  const float y = (0.5f * z) * (pos ? 2.0f - (shifted ? 0.0f : c) : c);  // erfc(-x) = 2 - erfc(x)
  return (shifted && !pos) ? y * 0x1p-64f : y;
}

__device__ __forceinline__ float gelu_tanh(float z) {
#pragma clang fp contract(off)
  const float z3 = (z * z) * z;
  const float t = 0.797884560802865355f * (z + 0.044715f * z3);   // sqrt(2/pi)
  const float q = (-2.0f * kLog2e) * __builtin_fabsf(t);
  const bool shifted = q < -64.0f;
  const float e = __builtin_amdgcn_exp2f(shifted ? q + 64.0f : q);     // exp(-2|t|) (* 2^64)
  const float r = __builtin_amdgcn_rcpf(1.0f + (shifted ? 0.0f : e));
  const bool pos = t >= 0.0f;
  const float y = (pos ? z : z * e) * r;
  return (shifted && !pos) ? y * 0x1p-64f : y;
}

// Adds the WPR per-wave values of this wave's row in part order (the same
// order in every wave of the row); `slot` is this workgroup's LDS array.
template <int WPR>
__device__ __forceinline__ float row_sum_parts(float v, float* slot, int wave, int lane) {
  if constexpr (WPR == 1) {
    return v;
  } else {
    if (lane == 0) slot[wave] = v;
    lds_barrier();
    const int base = wave - wave % WPR;
    float s = slot[base];
#pragma unroll
    for (int p = 1; p < WPR; ++p) s = s + slot[base + p];
    return s;
  }
}

template <int WPR>
__device__ __forceinline__ uint32_t row_max_parts(uint32_t v, uint32_t* slot, int wave, int lane) {
  if constexpr (WPR == 1) {
    return v;
  } else {
    if (lane == 0) slot[wave] = v;
    lds_barrier();
    const int base = wave - wave % WPR;
    uint32_t m = slot[base];
#pragma unroll
    for (int p = 1; p < WPR; ++p) m = max(m, slot[base + p]);
    return m;
  }
}

template <int OP, int CH, int WPR>
__global__ __launch_bounds__(256) void producer_quant_kernel(ProducerArgs a) {
  static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
  constexpr int RPB = 4 / WPR;                       // rows per workgroup
  __shared__ float red_sum[4];
  __shared__ float red_sq[4];
  __shared__ uint32_t red_max[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
  const bool valid = row < a.M;
  if (WPR == 1 && !valid) return;
  const uint32_t nchunks = (uint32_t)(a.K >> 3);
  const uint32_t row_bytes = valid ? (uint32_t)a.K * 2u : 0u;   // past the last row: reads zero
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (valid ? row : 0) * a.ldx, row_bytes);

  uint4 v[CH];
  uint4 sh[OP == kProducerLayerNorm ? CH : 1];
  uint4 sc[OP == kProducerLayerNorm ? CH : 1];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = load16_nt(rx, (uint32_t)(lane + 64 * (part + WPR * c)) * 16u);
  if constexpr (OP == kProducerLayerNorm) {
    const int64_t g = (valid ? row : 0) / a.rows_per_group;
    const __amdgpu_buffer_rsrc_t rsh = make_rsrc(a.shift + g * a.ld_mod, row_bytes);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.scale + g * a.ld_mod, row_bytes);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t off = (uint32_t)(lane + 64 * (part + WPR * c)) * 16u;
      sh[c] = load16(rsh, off);
      sc[c] = load16(rsc, off);
    }
  }

  // the producer's row y in fp32, then rounded to bf16 in place of x. The
  // row's amax is taken on the fp32 values: rounding to nearest even is
  // monotone and odd, so max |bf16(y)| = bf16(max |y|).
  float amaxf = 0.0f;
  if constexpr (OP == kProducerLayerNorm) {
#pragma clang fp contract(off)
    float f[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) unpack8(v[c], f[c]);
    // chunks past K read zero and add nothing to the sum
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) s = s + f[c][i];
    s = row_sum_parts<WPR>(wave_sum(s), red_sum, wave, lane);
    const float mean = s / (float)a.K;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * (part + WPR * c) < (int)nchunks) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = f[c][i] - mean;
          q = __builtin_fmaf(d, d, q);
        }
      }
    }
    q = row_sum_parts<WPR>(wave_sum(q), red_sq, wave, lane);
    const float rstd = 1.0f / __builtin_sqrtf(q / (float)a.K + a.eps);
    const float nmr = -(mean * rstd);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * (part + WPR * c) < (int)nchunks) {
        float fs[8], fh[8];
        unpack8(sc[c], fs);
        unpack8(sh[c], fh);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = __builtin_fmaf(f[c][i], rstd, nmr);          // (x - mean) rstd
          f[c][i] = __builtin_fmaf(t, 1.0f + fs[i], fh[i]);
          amaxf = __builtin_fmaxf(amaxf, __builtin_fabsf(f[c][i]));
        }
        v[c] = pack8_bf16(f[c]);
      } else {
        v[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  } else {
    // chunks past K read zero, and GELU(0) = 0 in both forms
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float f[8];
      unpack8(v[c], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f[i] = OP == kProducerGelu ? gelu_erf(f[i]) : gelu_tanh(f[i]);
        amaxf = __builtin_fmaxf(amaxf, __builtin_fabsf(f[i]));
      }
      v[c] = pack8_bf16(f);
    }
  }

  // per-row quantisation of the bf16 row (the activation quantisation's maths)
  uint32_t amax = f32_to_bf16_rne(amaxf);
  amax = row_max_parts<WPR>(wave_max_u32(amax), red_max, wave, lane);
  if (!valid) return;
  const float s = row_scale<false>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;   // subnormal scale
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.xq + row * a.K, (uint32_t)a.K);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t idx = (uint32_t)(lane + 64 * (part + WPR * c));
    store8(quant8<false>(v[c], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
  }
  if (a.y) {
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y + row * a.ldy, (uint32_t)a.K * 2u);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t idx = (uint32_t)(lane + 64 * (part + WPR * c));
      store16(v[c], ry, idx < nchunks ? idx * 16u : kOOB);
    }
  }
  if (lane == 0 && part == 0) a.a_scale[row] = s;
}

// z -> bf16(GELU(z)) for every bf16 bit pattern z, erf form then tanh form.
__device__ __attribute__((aligned(16))) uint16_t g_gelu_table[2][65536];

constexpr int kLutWaves = 16;                        // waves per lookup workgroup
constexpr size_t kLutBytes = 65536 * sizeof(uint16_t);

template <int OP>
__global__ __launch_bounds__(256) void gelu_table_kernel() {
  const uint32_t z = blockIdx.x * 256u + threadIdx.x;          // grid 256 x 256
  const float zf = bf16_to_f32(z);
  const float y = OP == kProducerGelu ? gelu_erf(zf) : gelu_tanh(zf);
  g_gelu_table[OP - kProducerGelu][z] =
      (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){y, 0.0f}, v2bf));
}

// WPR waves per row (wave part p holds chunks lane + 64 (p + WPR c), c < CH),
// 16 / WPR rows per iteration of the workgroup. Each wave requests its part
// of the row DEPTH iterations ahead before it works on the current one, so
// DEPTH + 1 rows per wave stay in flight; the parts of a row exchange their
// amax through LDS slots, double-buffered by iteration so one barrier per
// iteration suffices (no wave runs more than one iteration ahead of
// another). Every wave of a workgroup runs the same number of iterations; a
// row past M reads zero and stores nothing.
template <int OP, int CH, int WPR, int DEPTH>
__global__ __launch_bounds__(64 * kLutWaves) void gelu_lut_quant_kernel(ProducerArgs a) {
  static_assert(WPR == 4 || WPR == 8 || WPR == 16, "waves per row");
  static_assert(DEPTH == 1 || DEPTH == 2, "rows requested ahead");
  constexpr int RPI = kLutWaves / WPR;               // rows per iteration
  extern __shared__ __attribute__((aligned(16))) uint16_t lut[];
  __shared__ uint32_t part_max[2][kLutWaves];
  {
    const uint4* src = reinterpret_cast<const uint4*>(g_gelu_table[OP - kProducerGelu]);
    uint4* dst = reinterpret_cast<uint4*>(lut);
    constexpr int kPer = (int)(kLutBytes / 16) / (64 * kLutWaves);
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[threadIdx.x + 64 * kLutWaves * i] = src[threadIdx.x + 64 * kLutWaves * i];
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % WPR;
  // byte offset of the lane's first chunk in a row; every offset is in the
  // vector offset, which the descriptor bound checks, so chunks past K load
  // zero and their stores are dropped
  const uint32_t off0 = (uint32_t)(lane + 64 * part) * 16u;
  constexpr uint32_t kStep = 1024u * WPR;            // bytes between a lane's chunks
  const int64_t stride = (int64_t)gridDim.x * RPI;

  auto load_row = [&](int64_t row, uint4 (&dst)[CH]) {
    const bool in = row < a.M;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(a.x + (in ? row : 0) * a.ldx, in ? (uint32_t)a.K * 2u : 0u);
#pragma unroll
    for (int c = 0; c < CH; ++c) dst[c] = load16_nt(rx, off0 + kStep * c);
  };
  int64_t row = (int64_t)blockIdx.x * RPI + wave / WPR;
  uint4 b[DEPTH + 1][CH];                            // b[0]: this iteration's row
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_row(row + d * stride, b[d]);
  __syncthreads();                                  // the table is in LDS
  for (int k = 0; (int64_t)blockIdx.x * RPI + k * stride < a.M; ++k, row += stride) {
    load_row(row + DEPTH * stride, b[DEPTH]);
    uint4 (&v)[CH] = b[0];
    const bool in = row < a.M;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y + (in ? row : 0) * a.ldy,
                                                (a.y && in) ? (uint32_t)a.K * 2u : 0u);
    // the table maps 0 (a chunk past K) to 0
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = (uint32_t)lut[w[i] & 0xffffu] | ((uint32_t)lut[w[i] >> 16] << 16);
        // the packed pair exists before the y store's branch (else both
        // halves of every chunk stay live until the quantisation)
        asm volatile("" : "+v"(w[i]));
      }
      v[c] = make_uint4(w[0], w[1], w[2], w[3]);
      amax = absmax_bits8(v[c], amax);
      if (a.y) store16(v[c], ry, off0 + kStep * c);
    }
    amax = wave_max_u32(amax);
    if (lane == 0) part_max[k & 1][wave] = amax;
    lds_barrier();
    const int base = wave - part;
#pragma unroll
    for (int p = 0; p < WPR; ++p) amax = max(amax, part_max[k & 1][base + p]);
    if (in) {
      const float s = row_scale<false>(amax);
      const bool zero = (amax == 0);
      const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;   // subnormal scale
      const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.xq + row * a.K, (uint32_t)a.K);
#pragma unroll
      for (int c = 0; c < CH; ++c)
        store8(quant8<false>(v[c], s, r, zero, exact_div), rq, (off0 >> 1) + (kStep >> 1) * c);
      if (lane == 0 && part == 0) a.a_scale[row] = s;
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int c = 0; c < CH; ++c) b[d][c] = b[d + 1][c];
  }
}

template <int OP, int CH, int WPR, int DEPTH>
hipError_t launch_lut(const ProducerArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gelu_table_kernel<OP>), dim3(256), dim3(256), 0, stream);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  constexpr int RPI = kLutWaves / WPR;
  const int64_t wgs_needed = (a.M + RPI - 1) / RPI;
  const int64_t cus = device_cus();
  const unsigned grid = (unsigned)(wgs_needed < cus ? wgs_needed : cus);
  hipLaunchKernelGGL((gelu_lut_quant_kernel<OP, CH, WPR, DEPTH>), dim3(grid), dim3(64 * kLutWaves),
                     kLutBytes, stream, a);
  return hipGetLastError();
}

// The table path pays for its table build (65536 evaluations) from about
// 4 M elements on; 4 or 16 waves hold a row, at most 2 chunks per lane
// (rows up to K = 16384 take it).
constexpr int64_t kLutMinElements = int64_t(1) << 22;
constexpr int64_t kLutMaxChunks = 2048;

template <int OP>
hipError_t launch_gelu_lut(const ProducerArgs& a, hipStream_t stream) {
  // waves per row, rows requested ahead: at 4352 x 12288, 4 and 1 ran in
  // 45 us, 8 and 1 in 50 us, 16 and 2 in 57 us (wider rows mean more waves
  // at each barrier; deeper prefetch, more register moves)
  constexpr int W = 4, D = 1;
  const int64_t per_lane = ((a.K >> 3) + 64 * W - 1) / (64 * W);
  if (per_lane <= 1) return launch_lut<OP, 1, W, D>(a, stream);
  if (per_lane <= 2) return launch_lut<OP, 2, W, D>(a, stream);
  if (per_lane <= 4) return launch_lut<OP, 4, W, D>(a, stream);
  if (per_lane <= 6) return launch_lut<OP, 6, W, D>(a, stream);
  return launch_lut<OP, 8, W, D>(a, stream);
}

template <int OP, int CH, int WPR>
hipError_t launch_cfg(const ProducerArgs& a, hipStream_t stream) {
  constexpr int RPB = 4 / WPR;
  hipLaunchKernelGGL((producer_quant_kernel<OP, CH, WPR>), dim3((unsigned)((a.M + RPB - 1) / RPB)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int OP>
hipError_t launch_op(const ProducerArgs& a, hipStream_t stream) {
  const int64_t nchunks = a.K >> 3;
  if constexpr (OP != kProducerLayerNorm) {
    if (nchunks <= kLutMaxChunks && a.M * a.K >= kLutMinElements) return launch_gelu_lut<OP>(a, stream);
  }
  if (nchunks <= 64) return launch_cfg<OP, 1, 1>(a, stream);
  if (nchunks <= 128) return launch_cfg<OP, 2, 1>(a, stream);
  if (nchunks <= 256) return launch_cfg<OP, 2, 2>(a, stream);
  if (nchunks <= 384) return launch_cfg<OP, 3, 2>(a, stream);
  if (nchunks <= 512) return launch_cfg<OP, 4, 2>(a, stream);
  if (nchunks <= 1024) return launch_cfg<OP, 4, 4>(a, stream);
  if (nchunks <= 1536) return launch_cfg<OP, 6, 4>(a, stream);
  if (nchunks <= 2048) return launch_cfg<OP, 8, 4>(a, stream);
  if constexpr (OP != kProducerLayerNorm) {
    if (nchunks <= 3072) return launch_cfg<OP, 12, 4>(a, stream);
    if (nchunks <= 4096) return launch_cfg<OP, 16, 4>(a, stream);
  }
  return hipErrorInvalidValue;      // past kProducerMaxK: rejected before the launch
}

}  // namespace

hipError_t launch_producer_quant(const ProducerArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  switch (a.op) {
    case kProducerLayerNorm: return launch_op<kProducerLayerNorm>(a, stream);
    case kProducerGelu: return launch_op<kProducerGelu>(a, stream);
    case kProducerGeluTanh: return launch_op<kProducerGeluTanh>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
