// Small-M W8A8 linear (M <= 16): one fused, weight-streaming kernel (gfx950).
//
// The int8 matmul route of the prior art requires more than 16 activation
// rows, so the AdaLN modulation and conditioning projections, which run at
// M = batch = 1, were kept out of int8 (unsloth commit log of
// test_diffusion_transformer_quant.py). Here they are served by a kernel
// whose cost is streaming the int8 weight once from HBM.
//
// Per workgroup (256 threads, one per CU for the usual N):
//  1. quantise the M activation rows on chip (per-row amax, scale =
//     amax/127, exact half-to-even rounding) into LDS as int8 [16][K];
//     rows M..15 are never stored, since their output columns are discarded;
//     workgroup 0 also writes xq and a_scale out for the caller.
//  2. stream a contiguous range of weight rows: each 16-row block is the
//     MFMA "A" operand of v_mfma_i32_16x16x64_i8, loaded straight from HBM
//     into registers (16 bytes per lane), the activations are the "B"
//     operand read from LDS. The four waves split K; loads are software
//     pipelined one batch ahead.
//  3. reduce the four K-partials of every block through LDS (int32, exact)
//     and apply the same epilogue as the GEMM, so a row gives bit-identical
//     results on either path.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kMaxBlocks = 6;                 // 16-row weight blocks per workgroup
constexpr int kXsStride = kSmallMMaxK + 16;   // LDS row stride (bank spread)
constexpr int kU = 4;                         // k-steps (64 bytes each) per load batch

template <bool HAS_BIAS>
__global__ __launch_bounds__(256) void small_m_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                      GemmArgs a, int rows_per_wg, int kw,
                                                      int8_t* __restrict__ xq_out,
                                                      float* __restrict__ sa_out, int vec_flags) {
  __shared__ __attribute__((aligned(16))) int8_t xs[16 * kXsStride];
  __shared__ float sa_lds[16];
  __shared__ v4i red[kMaxBlocks][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t row_end = min(N, row_begin + rows_per_wg);
  const int nblk = (int)((row_end - row_begin + 15) / 16);

  // This wave's k-steps: [k_lo, k_lo + kw); steps at or past K load zeros.
  const int k_lo = wave * kw;
  const int nbatch_per_blk = kw / kU;
  const int nbatch = nblk * nbatch_per_blk;
  const int frag_row = lane & 15, frag_grp = lane >> 4;

  auto load_batch = [&](int i, v4i* f) {
    const int b = i / nbatch_per_blk, kb = i % nbatch_per_blk;
    const int64_t n = row_begin + 16 * b + frag_row;
    const bool nval = n < row_end;
    const int8_t* base = a.wq + n * K + 16 * frag_grp;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t kbyte = (int64_t)(k_lo + kb * kU + u) * 64;
      f[u] = (nval && kbyte + 16 * frag_grp < K)
                 ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + kbyte))
                 : v4i{0, 0, 0, 0};
    }
  };

  v4i f0[kU], f1[kU];
  if (nbatch > 0) load_batch(0, f0);

  // ---- 1. activation quantisation into LDS ----
  const int nchunks = (int)(K >> 3);
  for (int m = wave; m < M; m += 4) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)m * ldx);
    uint32_t amax = 0;
    for (int idx = lane; idx < nchunks; idx += 64) amax = absmax_bits8(src[idx], amax);
    amax = wave_max_u32(amax);
    const float s = row_scale(amax);
    const bool zero = (amax == 0);
    const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
    const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
    for (int idx = lane; idx < nchunks; idx += 64) {
      const uint2 q = quant8(src[idx], s, r, zero, exact_div);
      *reinterpret_cast<uint2*>(&xs[m * kXsStride + 8 * idx]) = q;
      if (blockIdx.x == 0) *reinterpret_cast<uint2*>(xq_out + (int64_t)m * K + 8 * idx) = q;
    }
    if (lane == 0) {
      sa_lds[m] = s;
      if (blockIdx.x == 0) sa_out[m] = s;
    }
  }
  __syncthreads();

  // ---- 2. weight streaming ----
  v4i acc = v4i{0, 0, 0, 0};
  for (int i = 0; i < nbatch; ++i) {
    if (i + 1 < nbatch) load_batch(i + 1, f1);
    const int kb = i % nbatch_per_blk;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kstep = k_lo + kb * kU + u;
      // k-steps past K multiply zero weights; clamp the LDS read in bounds.
      const int kbyte = min(kstep * 64, kSmallMMaxK - 64);
      const v4i fx = *reinterpret_cast<const v4i*>(&xs[frag_row * kXsStride + kbyte + 16 * frag_grp]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0[u], fx, acc, 0, 0, 0);
    }
    if (kb == nbatch_per_blk - 1) {
      red[i / nbatch_per_blk][wave][lane] = acc;
      acc = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) f0[u] = f1[u];
  }
  __syncthreads();

  // ---- 3. K-partial reduction and epilogue ----
  const int m = lane & 15;
  if (m >= M) return;
  const float sa = sa_lds[m];
  for (int b = wave; b < nblk; b += 4) {
    const v4i c = red[b][0][lane] + red[b][1][lane] + red[b][2][lane] + red[b][3][lane];
    const int64_t n = row_begin + 16 * b + 4 * (lane >> 4);
    if (n >= row_end) continue;
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (n + r < row_end) {
        const float bb = HAS_BIAS ? bf16_to_f32(a.bias[n + r]) : 0.f;
        y[r] = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(c[r], sa, a.w_scale[n + r], bb));
      } else {
        y[r] = 0;
      }
    }
    uint16_t* o = a.out + (int64_t)m * a.ldo + n;
    if (n + 3 < row_end && (vec_flags & 1)) {
      *reinterpret_cast<uint2*>(o) = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < row_end) o[r] = (uint16_t)y[r];
    }
    if (a.acc_debug) {
      int32_t* d = a.acc_debug + (int64_t)m * N + n;
      if (n + 3 < row_end && (vec_flags & 2)) {
        *reinterpret_cast<int4*>(d) = make_int4(c[0], c[1], c[2], c[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < row_end) d[r] = c[r];
      }
    }
  }
}

}  // namespace

hipError_t launch_small_m(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  // Rows per workgroup: spread N over ~256 workgroups (one per CU), in
  // multiples of 8 rows, at most kMaxBlocks 16-row blocks.
  int64_t rows = (a.N + 255) / 256;
  rows = ((rows + 7) / 8) * 8;
  if (rows > 16 * kMaxBlocks) rows = 16 * kMaxBlocks;
  const int64_t grid = (a.N + rows - 1) / rows;
  // k-steps of 64 bytes, split over 4 waves, rounded up to whole batches.
  const int64_t ksteps = (a.K + 63) / 64;
  int64_t kw = (ksteps + 3) / 4;
  kw = ((kw + kU - 1) / kU) * kU;
  const int vec_flags = epilogue_vec_flags(a);
  if (a.bias)
    hipLaunchKernelGGL(small_m_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, a,
                       (int)rows, (int)kw, xq_out, a_scale_out, vec_flags);
  else
    hipLaunchKernelGGL(small_m_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, a,
                       (int)rows, (int)kw, xq_out, a_scale_out, vec_flags);
  return hipGetLastError();
}

}  // namespace w8a8
