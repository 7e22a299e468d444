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
// waves per row (from K = 1024 and K = 4096 on), lane `lane` of wave part p
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
//   K / 64 + 16 additions. mean = sum / K, var = (sum of (x - mean)^2) / K,
//   rstd = 1 / sqrt(var + eps), y = ((x - mean) * rstd) * (1 + scale) + shift.
//   GELU: (0.5 z) * erfc(-z / sqrt 2), which has no cancellation for z << 0.
//   tanh form: with t = sqrt(2/pi) (z + 0.044715 z^3) and e = exp(-2|t|),
//   z / (1 + e) for t >= 0 and z e / (1 + e) for t < 0 (the same function as
//   0.5 z (1 + tanh t), without the overflow of exp(-2t) at t << 0).
#include "producers.h"
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

__device__ __forceinline__ uint4 pack8_bf16(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(f[2 * i]) | (f32_to_bf16_rne(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float gelu_erf(float z) {
#pragma clang fp contract(off)
  const float a = z * -0.707106781186547524f;     // -z / sqrt 2
  return (0.5f * z) * erfcf(a);
}

__device__ __forceinline__ float gelu_tanh(float z) {
#pragma clang fp contract(off)
  const float z3 = (z * z) * z;
  const float t = 0.797884560802865355f * (z + 0.044715f * z3);   // sqrt(2/pi)
  const float e = expf(-2.0f * __builtin_fabsf(t));
  const float den = 1.0f + e;
  return t >= 0.0f ? z / den : (z * e) / den;
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

  // the producer's bf16 row, in place of x
  if constexpr (OP == kProducerLayerNorm) {
#pragma clang fp contract(off)
    // chunks past K read zero and add nothing to the sum
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float f[8];
      unpack8(v[c], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) s = s + f[i];
    }
    s = row_sum_parts<WPR>(wave_sum(s), red_sum, wave, lane);
    const float mean = s / (float)a.K;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * (part + WPR * c) < (int)nchunks) {
        float f[8];
        unpack8(v[c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = f[i] - mean;
          q = q + d * d;
        }
      }
    }
    q = row_sum_parts<WPR>(wave_sum(q), red_sq, wave, lane);
    const float rstd = 1.0f / __builtin_sqrtf(q / (float)a.K + a.eps);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * (part + WPR * c) < (int)nchunks) {
        float f[8], fs[8], fh[8];
        unpack8(v[c], f);
        unpack8(sc[c], fs);
        unpack8(sh[c], fh);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float t = f[i] - mean;
          t = t * rstd;
          t = t * (1.0f + fs[i]);
          f[i] = t + fh[i];
        }
        v[c] = pack8_bf16(f);
      } else {
        v[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * (part + WPR * c) < (int)nchunks) {
        float f[8];
        unpack8(v[c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = OP == kProducerGelu ? gelu_erf(f[i]) : gelu_tanh(f[i]);
        v[c] = pack8_bf16(f);
      } else {
        v[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  // per-row quantisation of the bf16 row (the activation quantisation's maths)
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) amax = absmax_bits8(v[c], amax);
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
