// Small-M W8A8 linear (M <= 32): one fused, weight-streaming kernel (gfx950).
// Activations, bias and output are bf16, or all fp16 (same arithmetic).
//
// The int8 matmul route of the prior art requires more than 16 activation
// rows, so the AdaLN modulation and conditioning projections, which run at
// M = batch = 1, were kept out of int8 (unsloth commit log of
// test_diffusion_transformer_quant.py). Here they are served by a kernel
// whose cost is streaming the int8 weight once from HBM.
//
// Workgroups of W waves (4..12, one workgroup per CU when the weight allows;
// see row_groups.h), each wave owning 8 weight rows over the whole K, read in
// 128-byte windows:
//  1. the M activation rows are quantised on chip (per-row amax, scale =
//     amax/127, exact half-to-even rounding) into LDS as int8 [M][K];
//     workgroup 0 also writes xq and a_scale out for the caller. The rows
//     are requested before any weight window (vector-memory requests of the
//     whole chip share the same queues, and the few KiB of x requested behind
//     the weight stream would arrive last); the windows follow at once. With M <= W (at most one
//     row per wave) the quantisation itself then runs while the weights
//     stream;
//  2. the wave requests up to kD 128-byte windows of its rows at once
//     (one buffer_load_dwordx4 per window: lane l reads row l%8, 16-byte
//     chunk l/8, so every instruction fetches 8 whole 128-byte lines).
//     Each window is one v_mfma_i32_16x16x64_i8 per block of 8 tokens (up
//     to 4 blocks). The loaded
//     layout is the MFMA "A" layout if A-row i is read as weight row i%8 at
//     chunk parity i/8: lane l holds A[l%16][k-group l/16] = row l%8, chunk
//     2*(l/16) + (l/8)%2 = l/8. The "B" operand is built the same way from
//     LDS: column j = token j%8 at chunk parity j/8. Then
//     D[n][t] + D[n+8][t+8] is the dot product of weight row n and token t
//     over the window (the other two blocks of D are unused). The loads are
//     refilled kD windows ahead through a buffer descriptor bounded at the
//     wave's rows, so rows past N and chunks past K read as zero, branch-free;
//  3. the epilogue is the GEMM's, in the same fp32 order, so a row gives
//     bit-identical results on either path.
#include "row_groups.h"
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kD = 24;                   // 128-byte windows in flight per wave
constexpr int kQ = 6;                    // 16-byte chunks per lane per quantisation batch
constexpr int64_t kShortK = 128 * kD;    // K up to this: every window in flight at once

// Work split of a launch: ONE_ROW: M <= W and K <= kShortK (a wave quantises
// at most one activation row, overlapped with the weight stream); TWO_ROWS:
// the same with up to two rows per wave (M <= 2W, M <= 16, bf16); SHORT: K <=
// kShortK, rows quantised before the stream; LONG: longer rows (read twice
// for quantisation, weight windows refilled as they are consumed). Above 16
// rows (four token blocks) only SHORT and LONG are used.
enum Mode { ONE_ROW = 0, SHORT = 1, LONG = 2, TWO_ROWS = 3 };

// LDS row stride for the quantised activations: K rounded up to whole
// 128-byte windows plus 32 bytes. One quarter-wave of the "B" read takes 8
// tokens x 2 adjacent 16-byte chunks; with the stride an odd multiple of 32
// modulo 256 after the padding (or 32 itself), those 16 chunks fall into 16
// distinct 16-byte bank groups.
__host__ __device__ inline int xs_stride(int64_t K) { return (int)((K + 127) / 128) * 128 + 32; }


// Quantises the row chunks held in v (chunk lane + 64*u of the row, u < Q)
// with the row's scale; returns the scale.
template <bool F16, int Q = kQ>
__device__ __forceinline__ float quantise_regs(const uint4 (&v)[Q], uint32_t nchunks, int lane,
                                               int8_t* xrow, int8_t* qrow, bool write_q) {
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < Q; ++u) amax = absmax_bits8(v[u], amax);
  amax = wave_max_u32(amax);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    if (64u * u >= nchunks) break;        // wave-uniform: no chunk of this batch is in the row
    const uint32_t idx = lane + 64 * u;
    const uint2 q = quant8<F16>(v[u], s, r, zero, exact_div);
    if (idx < nchunks) {
      *reinterpret_cast<uint2*>(xrow + 8 * idx) = q;
      if (write_q) *reinterpret_cast<uint2*>(qrow + 8 * idx) = q;
    }
  }
  return s;
}

// Rows longer than 64*kQ chunks: an amax pass, then a quantise pass that
// reads the row again.
template <bool F16>
__device__ __forceinline__ float quantise_long(__amdgpu_buffer_rsrc_t rx, uint32_t nchunks, int lane,
                                               int8_t* xrow, int8_t* qrow, bool write_q) {
  constexpr int U = 8;
  uint32_t amax = 0;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) amax = absmax_bits8(w[u], amax);
  }
  amax = wave_max_u32(amax);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      const uint2 q = quant8<F16>(w[u], s, r, zero, exact_div);
      if (idx < nchunks) {
        *reinterpret_cast<uint2*>(xrow + 8 * idx) = q;
        if (write_q) *reinterpret_cast<uint2*>(qrow + 8 * idx) = q;
      }
    }
  }
  return s;
}

// Up to kMaxWaves waves per workgroup: three waves per SIMD. TB: blocks of 8
// tokens (1, 2 or 4).
template <bool HAS_BIAS, int TB, int MODE, bool F16>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(3, 8))) void small_m_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, GemmArgs a, int8_t* __restrict__ xq_out,
    float* __restrict__ sa_out, int vec_flags, int G) {
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  __shared__ float sa_lds[8 * TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = blockDim.x >> 6;
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int ldxs = xs_stride(K);
  const int nwin = (int)((K + 127) / 128);
  // waves G.. of the workgroup own no weight rows: they only help quantise
  const int64_t n_base = ((int64_t)blockIdx.x * G + wave) * 8;
  const int rows_valid = wave < G ? (int)max<int64_t>(0, min<int64_t>(8, N - n_base)) : 0;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const bool write_q = blockIdx.x == 0;

  // weight windows: lane l reads row l%8, 16-byte chunk l/8 of window w
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.wq + (rows_valid > 0 ? n_base : 0) * K, (uint32_t)rows_valid * (uint32_t)K);
  const int chunk = lane >> 3;
  const uint32_t lane_off = (uint32_t)(lane & 7) * (uint32_t)K + 16u * chunk;
  auto wload = [&](int w) -> v4i {
    const bool in = 128 * w + 16 * chunk < K;          // chunks past K read as zero
    // non-temporal: the weight is streamed once; without the hint the loads
    // allocate in caches that a preceding write-heavy kernel left dirty, and
    // the stream waits on their write-back (measured: 21 against 14 us for
    // the 18432 x 3072 weight at M = 1 right after a DiT block)
    return __builtin_amdgcn_raw_buffer_load_b128(rw, in ? lane_off + 128u * w : kOOB, 0, 2);
  };
  v4i buf[kD];
  auto issue_all = [&]() {
#pragma unroll
    for (int d = 0; d < kD; ++d) buf[d] = wload(d);
    __builtin_amdgcn_sched_barrier(0);     // all requests out before the first use
  };

  // ---- 1. activation quantisation into LDS, 2. weight requests ----
  // The K tail of each LDS row up to whole windows is never written: it only
  // meets weights that read as zero. Token rows >= M give unused columns.
  if constexpr (MODE == ONE_ROW || MODE == TWO_ROWS) {
    // rows wave (and wave + W with TWO_ROWS) in registers across the weight
    // requests
    constexpr bool R2 = MODE == TWO_ROWS;
    const int m2 = wave + W;
    uint4 v[kQ], v2[R2 ? kQ : 1];
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)wave * ldx, (uint32_t)K * 2u);
    if (wave < M) {
#pragma unroll
      for (int u = 0; u < kQ; ++u) v[u] = load16(rx, (uint32_t)(lane + 64 * u) * 16u);
    }
    if constexpr (R2) {
      const __amdgpu_buffer_rsrc_t rx2 =
          make_rsrc(x + (int64_t)(m2 < M ? m2 : 0) * ldx, m2 < M ? (uint32_t)K * 2u : 0u);
#pragma unroll
      for (int u = 0; u < kQ; ++u) v2[u] = load16(rx2, (uint32_t)(lane + 64 * u) * 16u);
    }
    // the weight requests go out right behind the row loads; vmcnt(kD) then
    // waits for the rows only (loads complete in order)
    __builtin_amdgcn_sched_barrier(0);
    issue_all();
    wait_vmcnt<kD>();
    if (wave < M) {
      const float s = quantise_regs<F16>(v, nchunks, lane, xs + wave * ldxs, xq_out + (int64_t)wave * K,
                                    write_q);
      if (lane == 0) {
        sa_lds[wave] = s;
        if (write_q) sa_out[wave] = s;
      }
    }
    if constexpr (R2) {
      if (m2 < M) {
        const float s2 = quantise_regs<F16>(v2, nchunks, lane, xs + m2 * ldxs,
                                            xq_out + (int64_t)m2 * K, write_q);
        if (lane == 0) {
          sa_lds[m2] = s2;
          if (write_q) sa_out[m2] = s2;
        }
      }
    }
    lds_barrier();
  } else {
    for (int m = wave; m < M; m += W) {
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, (uint32_t)K * 2u);
      float s;
      if constexpr (MODE == SHORT) {
        uint4 v[kQ];
#pragma unroll
        for (int u = 0; u < kQ; ++u) v[u] = load16(rx, (uint32_t)(lane + 64 * u) * 16u);
        s = quantise_regs<F16>(v, nchunks, lane, xs + m * ldxs, xq_out + (int64_t)m * K, write_q);
      } else {
        s = quantise_long<F16>(rx, nchunks, lane, xs + m * ldxs, xq_out + (int64_t)m * K, write_q);
      }
      if (lane == 0) {
        sa_lds[m] = s;
        if (write_q) sa_out[m] = s;
      }
    }
    __syncthreads();
    if (rows_valid == 0) return;
    issue_all();
  }
  if (rows_valid == 0) return;

  // ---- 3. weight streaming ----
  v4i acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = v4i{0, 0, 0, 0};
  const int8_t* xb = xs + (lane & 7) * ldxs + 16 * chunk;
  // window w: its LDS read(s) and MFMA(s); windows past the end multiply zero
  // weights, so the LDS read is kept inside the row (its last window)
  auto window = [&](int w, const v4i& wv) {
    const int wc = min(w, nwin - 1);
    v4i b[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) b[t] = *reinterpret_cast<const v4i*>(xb + 8 * t * ldxs + 128 * wc);
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, b[t], acc[t], 0, 0, 0);
  };
  if constexpr (MODE != LONG) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      window(d, buf[d]);
      __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
    }
  } else {
    for (int base = 0; base < nwin; base += kD) {
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        window(base + d, buf[d]);
        buf[d] = wload(base + d + kD);
        __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  }

  // ---- 4. epilogue ----
  // D[i][j] sits in lane 16*(i/4) + j, element i%4. Row n < 8 at token t < 8
  // is D[n][t] + D[n+8][t+8], whose second term is 40 lanes up; lanes 0-7
  // and 16-23 then hold rows nl..nl+3 (nl = 4*(lane/16)) of token lane%8.
  const int src = ((lane + 40) & 63) * 4;
  v4i sum[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[t][r] = acc[t][r] + __builtin_amdgcn_ds_bpermute(src, acc[t][r]);
  if ((lane & 8) != 0 || lane >= 32) return;
  const int nl = 4 * (lane >> 4);
  const int64_t n = n_base + nl;
  float sw[4], bb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = nl + r < rows_valid;
    sw[r] = ok ? a.w_scale[n + r] : 0.f;
    bb[r] = (HAS_BIAS && ok) ? half_to_f32<F16>(a.bias[n + r]) : 0.f;
  }
#pragma unroll
  for (int blk = 0; blk < TB; ++blk) {
    const int m = 8 * blk + (lane & 7);
    if (m >= M) continue;
    const v4i c = sum[blk];
    const float sa = sa_lds[m];
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = f32_to_half_rne<F16>(epilogue_f32<HAS_BIAS>(c[r], sa, sw[r], bb[r]));
    uint16_t* o = a.out + (int64_t)m * a.ldo + n;
    if (nl + 3 < rows_valid && (vec_flags & 1)) {
      *reinterpret_cast<uint2*>(o) = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nl + r < rows_valid) o[r] = (uint16_t)y[r];
    }
    if (a.acc_debug) {
      int32_t* dst = a.acc_debug + (int64_t)m * N + n;
      if (nl + 3 < rows_valid && (vec_flags & 2)) {
        *reinterpret_cast<int4*>(dst) = make_int4(c[0], c[1], c[2], c[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nl + r < rows_valid) dst[r] = c[r];
      }
    }
  }
}

template <bool HAS_BIAS, int TB, bool F16>
hipError_t launch_variant(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  const RowGroupGrid g = row_group_grid(a.N);
  // Above 8 rows, kMaxWaves waves quantise the rows whatever the weight rows
  // per workgroup (g.waves groups), so the per-workgroup quantisation has
  // three waves per SIMD to hide its latency and spread its VALU work.
  const int threads = 64 * (TB >= 2 ? kMaxWaves : g.waves);
  const dim3 grid(g.blocks), block(threads);
  const int G = g.waves;
  const size_t lds = (size_t)(8 * TB) * (size_t)xs_stride(a.K);
  const int vf = epilogue_vec_flags(a);
  if (a.K > kShortK)
    hipLaunchKernelGGL((small_m_kernel<HAS_BIAS, TB, LONG, F16>), grid, block, lds, stream, x, ldx,
                       a, xq_out, a_scale_out, vf, G);
  else if (TB == 4)
    hipLaunchKernelGGL((small_m_kernel<HAS_BIAS, TB, SHORT, F16>), grid, block, lds, stream, x, ldx,
                       a, xq_out, a_scale_out, vf, G);
  else if (a.M <= threads / 64) {
    if constexpr (TB < 4)
      hipLaunchKernelGGL((small_m_kernel<HAS_BIAS, TB, ONE_ROW, F16>), grid, block, lds, stream, x,
                         ldx, a, xq_out, a_scale_out, vf, G);
  } else if (!F16 && a.M <= 2 * (threads / 64)) {
    // (bf16 only: the fp16 instantiation of this mode spills registers)
    if constexpr (!F16 && TB < 4)
      hipLaunchKernelGGL((small_m_kernel<HAS_BIAS, TB, TWO_ROWS, F16>), grid, block, lds, stream,
                         x, ldx, a, xq_out, a_scale_out, vf, G);
  } else
    hipLaunchKernelGGL((small_m_kernel<HAS_BIAS, TB, SHORT, F16>), grid, block, lds, stream, x, ldx,
                       a, xq_out, a_scale_out, vf, G);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_dtype(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                        float* a_scale_out, hipStream_t stream) {
  if (a.bias) {
    if (a.M > 16) return launch_variant<true, 4, F16>(x, ldx, a, xq_out, a_scale_out, stream);
    return a.M > 8 ? launch_variant<true, 2, F16>(x, ldx, a, xq_out, a_scale_out, stream)
                   : launch_variant<true, 1, F16>(x, ldx, a, xq_out, a_scale_out, stream);
  }
  if (a.M > 16) return launch_variant<false, 4, F16>(x, ldx, a, xq_out, a_scale_out, stream);
  return a.M > 8 ? launch_variant<false, 2, F16>(x, ldx, a, xq_out, a_scale_out, stream)
                 : launch_variant<false, 1, F16>(x, ldx, a, xq_out, a_scale_out, stream);
}

}  // namespace

hipError_t launch_small_m(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.M > kSmallMWideRows || a.K > (a.M > 16 ? kSmallMWideMaxK : kSmallMMaxK))
    return hipErrorInvalidValue;
  return a.f16 ? launch_dtype<true>(x, ldx, a, xq_out, a_scale_out, stream)
               : launch_dtype<false>(x, ldx, a, xq_out, a_scale_out, stream);
}

}  // namespace w8a8
