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
// The LayerNorm kernel follows the quantisation kernels: one to four waves
// per row (two from K > 1024, or three up to K = 3072 when there are at
// most 1024 rows; four from K > 4096), lane `lane` of wave
// part p holding the row's 16-byte chunks lane + 64 (p + WPR c), c < CH, all
// requested at once (non-temporal: x is read once) and kept in registers
// through every step, so the row is read from HBM once and written once as
// int8. Chunks past K read zero through the bounded buffer descriptor and are
// masked out of the sums and the amax. Its fp32 evaluation (no contraction;
// correctly rounded division and square root): each lane sums its 8 CH
// values in order, a DPP reduction adds the lanes (six additions per term;
// one lane's total is used by every lane) and the WPR wave sums are added in
// part order: no term passes through more than K / 64 + 16 additions.
// mean = sum / K, var = (sum of (x - mean)^2) / K (squares accumulated by
// fused multiply-add), rstd = 1 / sqrt(var + eps),
// y = fma(fma(x, rstd, -(mean rstd)), 1 + scale, shift): two roundings fewer
// than the literal order, and the rounding of mean rstd is within the error
// the mean itself carries (u |mean| rstd). The bf16 rounding is
// v_cvt_pk_bf16_f32 (nearest even, subnormals kept).
//
// GELU goes through a table: a bf16 input has 65536 values, so the whole map
// z -> bf16(GELU(z)) is 128 KB, which fits in one compute unit's 160 KB of
// LDS. The map of each form is computed at build time in double precision
// and rounded once to the nearest bf16 (gen_gelu_table.cpp), and the library
// carries it as read-only data; nothing is computed or written for it at run
// time. The kernel copies it into LDS once per workgroup (one 1024-thread
// workgroup per compute unit, four rows at a time with four waves to a row,
// two rows with eight waves for rows of more than 16384 elements, or one
// row with all sixteen waves when there are at most 512 rows of up to 16384
// elements), and each element is one LDS lookup.
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

// Sum over the 64 lanes: DPP within rows of 16 (xor 1, xor 2 in quads, then
// rotations by 4 and 8), then lane 15 of each row into the next and lane 31
// into the upper half; every term passes through six additions (as in a
// butterfly) and the total is read from lane 63, so every lane returns the
// same value. Every lane must be active. (The DPP source of a row left out
// by the row mask reads 0, so those rows add nothing.)
__device__ __forceinline__ float wave_sum(float v) {
#define W8A8_DPP_ADD(ctrl, rows) \
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rows, 0xF, false))
  W8A8_DPP_ADD(0xB1, 0xF);     // quad [1,0,3,2]
  W8A8_DPP_ADD(0x4E, 0xF);     // quad [2,3,0,1]
  W8A8_DPP_ADD(0x124, 0xF);    // row_ror 4
  W8A8_DPP_ADD(0x128, 0xF);    // row_ror 8
  W8A8_DPP_ADD(0x142, 0xA);    // row_bcast 15
  W8A8_DPP_ADD(0x143, 0xC);    // row_bcast 31
#undef W8A8_DPP_ADD
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

// The modulated LayerNorm fused with the quantisation (OP is always
// kProducerLayerNorm: GELU takes the table kernel below).
template <int WPR>
constexpr int ln_rows_per_block() { return WPR == 3 ? 2 : 4 / WPR; }

template <int OP, int CH, int WPR>
__global__ __launch_bounds__(64 * WPR * ln_rows_per_block<WPR>()) void producer_quant_kernel(
    ProducerArgs a) {
  static_assert(OP == kProducerLayerNorm, "LayerNorm only");
  static_assert(WPR >= 1 && WPR <= 4, "waves per row");
  constexpr int RPB = ln_rows_per_block<WPR>();      // rows per workgroup
  __shared__ float red_sum[RPB * WPR];
  __shared__ float red_sq[RPB * WPR];
  __shared__ uint32_t red_max[RPB * WPR];
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
  uint4 sh[CH];
  uint4 sc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = load16_nt(rx, (uint32_t)(lane + 64 * (part + WPR * c)) * 16u);
  if constexpr (OP == kProducerLayerNorm) {
    // the row's modulation group: 32-bit division where both fit (the
    // 64-bit one is a long instruction sequence ahead of these loads)
    const uint64_t r64 = (uint64_t)(valid ? row : 0), rpg = (uint64_t)a.rows_per_group;
    const int64_t g = (r64 | rpg) >> 32 ? (int64_t)(r64 / rpg) : (int64_t)((uint32_t)r64 / (uint32_t)rpg);
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
  {
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

// z -> bf16(GELU(z)) for every bf16 bit pattern z, erf form then tanh form:
// read-only data, computed at build time in double precision and rounded
// once to the nearest bf16 (gen_gelu_table.cpp).
__device__ __attribute__((aligned(16))) const uint16_t g_gelu_table[2][65536] = {
#include "gelu_table.inc"
};

constexpr int kLutWaves = 16;                        // waves per lookup workgroup
constexpr size_t kLutBytes = 65536 * sizeof(uint16_t);

// WPR waves per row (wave part p holds chunks lane + 64 (p + WPR c), c < CH),
// 16 / WPR rows per iteration of the workgroup. Each wave requests its part
// of the next iteration's row before it works on the current one, into the
// other of two register buffers (the loop is unrolled by two, so the buffers
// swap by name: a register copy of a row still in flight would wait for it
// there); the parts of a row exchange their amax through LDS slots,
// double-buffered by iteration so one barrier per iteration suffices (no wave
// runs more than one iteration ahead of another). Iteration k of workgroup b
// (of G) takes rows k S + g G + b, S = G * 16 / WPR, for its row groups
// g = 0, 1, ...: a partial last sweep over M then gives every workgroup at
// most one row fewer than the others, rather than leaving the workgroups
// past its end idle. Every wave of a workgroup runs the same number of
// iterations (while its group 0 has a row); a row past M reads zero and
// stores nothing.
template <int OP, int CH, int WPR>
__global__ __launch_bounds__(64 * kLutWaves) void gelu_lut_quant_kernel(ProducerArgs a) {
  static_assert(WPR == 4 || WPR == 8 || WPR == 16, "waves per row");
  constexpr int RPI = kLutWaves / WPR;               // rows per iteration
  extern __shared__ __attribute__((aligned(16))) uint16_t lut[];
  __shared__ uint32_t part_max[2][kLutWaves];
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
  // iteration k on row `row` held in v
  auto process = [&](int k, int64_t row, uint4 (&v)[CH]) {
    const bool in = row < a.M;
    // every lookup of the part is requested before the first is used: one
    // LDS round trip for all of them (the table maps 0, a chunk past K, to 0)
    // (each pair is loaded into the two halves of one register)
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    v2u16 y2[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y2[c][i].x = lut[w[i] & 0xffffu];
        y2[c][i].y = lut[w[i] >> 16];
      }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      v[c] = make_uint4(__builtin_bit_cast(uint32_t, y2[c][0]), __builtin_bit_cast(uint32_t, y2[c][1]),
                        __builtin_bit_cast(uint32_t, y2[c][2]), __builtin_bit_cast(uint32_t, y2[c][3]));
      amax = absmax_bits8(v[c], amax);
    }
    if (a.y) {
      const __amdgpu_buffer_rsrc_t ry =
          make_rsrc(a.y + (in ? row : 0) * a.ldy, in ? (uint32_t)a.K * 2u : 0u);
#pragma unroll
      for (int c = 0; c < CH; ++c) store16(v[c], ry, off0 + kStep * c);
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
  };
  // iteration k runs while the workgroup's row of group 0 is below M
  auto live = [&](int k) { return (int64_t)blockIdx.x + k * stride < a.M; };
  int64_t row = (int64_t)blockIdx.x + (int64_t)(wave / WPR) * gridDim.x;
  uint4 b0[CH], b1[CH];
  // the first row is requested before the table: its HBM latency then
  // overlaps the table's copy from L2
  load_row(row, b0);
  {
    const uint4* src = reinterpret_cast<const uint4*>(g_gelu_table[OP - kProducerGelu]);
    uint4* dst = reinterpret_cast<uint4*>(lut);
    constexpr int kPer = (int)(kLutBytes / 16) / (64 * kLutWaves);
    uint4 t[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) t[i] = src[threadIdx.x + 64 * kLutWaves * i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[threadIdx.x + 64 * kLutWaves * i] = t[i];
  }
  __syncthreads();                                  // the table is in LDS
  for (int k = 0; live(k); k += 2, row += 2 * stride) {
    load_row(row + stride, b1);
    process(k, row, b0);
    if (!live(k + 1)) break;
    load_row(row + 2 * stride, b0);
    process(k + 1, row + stride, b1);
  }
}

template <int OP, int CH, int WPR>
hipError_t launch_lut(const ProducerArgs& a, hipStream_t stream) {
  constexpr int RPI = kLutWaves / WPR;
  const int64_t wgs_needed = (a.M + RPI - 1) / RPI;
  const int64_t cus = device_cus();
  const unsigned grid = (unsigned)(wgs_needed < cus ? wgs_needed : cus);
  hipLaunchKernelGGL((gelu_lut_quant_kernel<OP, CH, WPR>), dim3(grid), dim3(64 * kLutWaves),
                     kLutBytes, stream, a);
  return hipGetLastError();
}

// Every GELU call takes the table kernel: with the table built in, it
// measured faster than evaluating GELU per element at every size tried
// (16 to 1024 rows of 3072 and 12288 elements: 5.8-12.5 against 6.8-16.7 us
// per call), including one workgroup per four rows below a full chip.
template <int OP>
hipError_t launch_gelu_lut(const ProducerArgs& a, hipStream_t stream) {
  // waves per row: at 4352 x 12288, 4 ran in 45 us, 8 in 50 us, 16 in
  // 57 us (wider rows mean more waves at each barrier); rows of more than
  // 16384 elements take 8, so that a lane holds at most 8 chunks
  // up to 512 rows of up to 16384 elements: sixteen waves per row (one
  // row per workgroup iteration), so that few rows still spread over many
  // waves; per call, erf form, 16 / 64 / 256 / 512 rows of 12288 elements
  // 5.7 / 5.9 / 7.3 / 9.6 us against 9.2 / 9.8 / 11.7 / 12.6 with four, of
  // 3072 elements 4.4 / 4.5 / 4.7 / 5.9 against 5.4 / 6.0 / 6.0 / 6.3; at
  // 1024 rows equal (12288) or slower (3072: 8.7 against 6.6 us)
  if (a.M <= 512) {
    const int64_t p16 = ((a.K >> 3) + 1023) / 1024;
    if (p16 <= 1) return launch_lut<OP, 1, 16>(a, stream);
    if (p16 <= 2) return launch_lut<OP, 2, 16>(a, stream);
  }
  constexpr int W = 4;
  const int64_t per_lane = ((a.K >> 3) + 64 * W - 1) / (64 * W);
  if (per_lane <= 1) return launch_lut<OP, 1, W>(a, stream);
  if (per_lane <= 2) return launch_lut<OP, 2, W>(a, stream);
  if (per_lane <= 4) return launch_lut<OP, 4, W>(a, stream);
  if (per_lane <= 6) return launch_lut<OP, 6, W>(a, stream);
  if (per_lane <= 8) return launch_lut<OP, 8, W>(a, stream);
  const int64_t per_lane8 = ((a.K >> 3) + 64 * 8 - 1) / (64 * 8);
  if (per_lane8 <= 6) return launch_lut<OP, 6, 8>(a, stream);
  return launch_lut<OP, 8, 8>(a, stream);
}

template <int OP, int CH, int WPR>
hipError_t launch_cfg(const ProducerArgs& a, hipStream_t stream) {
  constexpr int RPB = ln_rows_per_block<WPR>();
  hipLaunchKernelGGL((producer_quant_kernel<OP, CH, WPR>), dim3((unsigned)((a.M + RPB - 1) / RPB)),
                     dim3(64 * WPR * RPB), 0, stream, a);
  return hipGetLastError();
}

template <int OP>
hipError_t launch_op(const ProducerArgs& a, hipStream_t stream) {
  if constexpr (OP != kProducerLayerNorm) {
    return launch_gelu_lut<OP>(a, stream);    // K <= 32768, checked before the launch
  } else {
    const int64_t nchunks = a.K >> 3;
    if (nchunks <= 64) return launch_cfg<OP, 1, 1>(a, stream);
    if (nchunks <= 128) return launch_cfg<OP, 2, 1>(a, stream);
    if (nchunks <= 256) return launch_cfg<OP, 2, 2>(a, stream);
    // rows of 2049-3072 elements: three waves per row (two chunks a lane)
    // while there are at most 1024 rows, two (three chunks) beyond. Per
    // call at K = 3072, 16 / 64 / 256 / 1024 rows: 4.5 / 4.5 / 4.8 / 6.4 us
    // against 5.0 / 5.4 / 5.6 / 6.7; equal at 1536 rows; 2048 / 3072 /
    // 4352 rows: 8.9 / 11.2 / 15.1 against 8.7 / 10.5 / 13.7 us
    if (nchunks <= 384) {
      if (a.M <= 1024) return launch_cfg<OP, 2, 3>(a, stream);
      return launch_cfg<OP, 3, 2>(a, stream);
    }
    if (nchunks <= 512) return launch_cfg<OP, 4, 2>(a, stream);
    if (nchunks <= 1024) return launch_cfg<OP, 4, 4>(a, stream);
    if (nchunks <= 1536) return launch_cfg<OP, 6, 4>(a, stream);
    if (nchunks <= 2048) return launch_cfg<OP, 8, 4>(a, stream);
    return hipErrorInvalidValue;    // past kProducerMaxK: rejected before the launch
  }
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
