// Small-M W8A8 linear (M <= 16): one fused, weight-streaming kernel (gfx950).
//
// The int8 matmul route of the prior art requires more than 16 activation
// rows, so the AdaLN modulation and conditioning projections, which run at
// M = batch = 1, were kept out of int8 (unsloth commit log of
// test_diffusion_transformer_quant.py). Here they are served by a kernel
// whose cost is streaming the int8 weight once from HBM.
//
// Workgroup of 4 waves, 64 weight rows; each wave owns 16 rows over the
// whole K:
//  0. the wave issues its first weight loads at once, so they are in flight
//     while the activations are quantised;
//  1. the M activation rows are quantised on chip (per-row amax, scale =
//     amax/127, exact half-to-even rounding) into LDS as int8 [16][K] (rows
//     M..15 are left unwritten: their output columns are discarded);
//     workgroup 0 also writes xq and a_scale out for the caller;
//  2. the wave streams its 16 weight rows: each 64-byte k-step of the 16
//     rows is the "A" operand of v_mfma_i32_16x16x64_i8, loaded straight from
//     HBM into registers through a bounded buffer descriptor (rows past N and
//     chunks past K read as zero, no branches), kDepth batches ahead; the
//     activations are the "B" operand, read from LDS;
//  3. the epilogue is the GEMM's, in the same fp32 order, so a row gives
//     bit-identical results on either path.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr uint32_t kOOB = 0x7ffffff0u;   // an offset past every descriptor bound
constexpr int kU = 4;                    // k-steps (64 bytes each) per load batch
constexpr int kDepth = 3;                // load batches in flight per wave
constexpr int kQ = 8;                    // 16-byte chunks per lane per quantisation batch

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// LDS row stride for the quantised activations: K rounded up to whole
// k-steps plus 16 bytes, an odd multiple of 16 modulo 256, so the 16 rows
// read by one ds_read_b128 land in distinct banks.
__host__ __device__ inline int xs_stride(int64_t K) {
  const int kp = (int)((K + 63) / 64) * 64;
  return kp + 16;
}

template <bool HAS_BIAS>
__global__ __launch_bounds__(256) void small_m_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                      GemmArgs a, int8_t* __restrict__ xq_out,
                                                      float* __restrict__ sa_out, int vec_flags) {
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  __shared__ float sa_lds[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int ldxs = xs_stride(K);
  const int64_t n_base = (int64_t)blockIdx.x * 64 + wave * 16;
  const int rows_valid = (int)max<int64_t>(0, min<int64_t>(16, N - n_base));

  // ---- 0. first weight batches ----
  const int ksteps = (int)((K + 63) / 64);
  const int nbatch = (ksteps + kU - 1) / kU;
  const int frag_row = lane & 15, frag_grp = lane >> 4;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.wq + (rows_valid > 0 ? n_base : 0) * K, (uint32_t)rows_valid * (uint32_t)K);
  const uint32_t lane_off = (uint32_t)frag_row * (uint32_t)K + 16u * frag_grp;
  auto load_batch = [&](int bi, v4i* f) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kb = (bi * kU + u) * 64 + 16 * frag_grp;     // this lane's K byte
      const uint32_t off = kb < K ? lane_off + (uint32_t)((bi * kU + u) * 64) : kOOB;
      f[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
    }
  };
  v4i f[kDepth][kU];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (d < nbatch) load_batch(d, f[d]);

  // ---- 1. activation quantisation into LDS ----
  // A wave per row; the row is read in batches of kQ x 16 bytes per lane,
  // all issued together (chunks past K read as zero through the bound).
  const uint32_t nchunks = (uint32_t)(K >> 3);
  for (int m = wave; m < M; m += 4) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, (uint32_t)K * 2u);
    uint32_t amax = 0;
    for (uint32_t base = 0; base < nchunks; base += 64 * kQ) {
      uint4 v[kQ];
#pragma unroll
      for (int u = 0; u < kQ; ++u) v[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
      for (int u = 0; u < kQ; ++u) amax = absmax_bits8(v[u], amax);
    }
    amax = wave_max_u32(amax);
    const float s = row_scale(amax);
    const bool zero = (amax == 0);
    const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
    const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
    for (uint32_t base = 0; base < nchunks; base += 64 * kQ) {
      uint4 v[kQ];
#pragma unroll
      for (int u = 0; u < kQ; ++u) v[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
      for (int u = 0; u < kQ; ++u) {
        const uint32_t idx = base + lane + 64 * u;
        if (idx < nchunks) {
          const uint2 q = quant8(v[u], s, r, zero, exact_div);
          *reinterpret_cast<uint2*>(&xs[m * ldxs + 8 * idx]) = q;
          if (blockIdx.x == 0) *reinterpret_cast<uint2*>(xq_out + (int64_t)m * K + 8 * idx) = q;
        }
      }
    }
    // the K tail of the row up to whole k-steps is read by the MFMAs against
    // zero weights; clear it so LDS holds defined values there
    for (int t = (int)K + 8 * lane; t < ldxs - 16; t += 512)
      *reinterpret_cast<uint2*>(&xs[m * ldxs + t]) = make_uint2(0u, 0u);
    if (lane == 0) {
      sa_lds[m] = s;
      if (blockIdx.x == 0) sa_out[m] = s;
    }
  }
  __syncthreads();
  if (rows_valid == 0) return;

  // ---- 2. weight streaming ----
  v4i acc = v4i{0, 0, 0, 0};
  const int8_t* xrow = xs + frag_row * ldxs + 16 * frag_grp;
  auto compute = [&](int bi, const v4i* fb) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // k-steps past the end multiply zero weights; keep the LDS read inside
      // the row (the last k-step of the padded row)
      const int ks = min(bi * kU + u, ksteps - 1);
      const v4i fx = *reinterpret_cast<const v4i*>(xrow + ks * 64);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[u], fx, acc, 0, 0, 0);
    }
  };
  int bi = 0;
  for (; bi + kDepth <= nbatch; bi += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      compute(bi + d, f[d]);
      if (bi + d + kDepth < nbatch) load_batch(bi + d + kDepth, f[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (bi + d < nbatch) compute(bi + d, f[d]);

  // ---- 3. epilogue: lane holds D[n = n_base + 4*(lane/16) + r][m = lane%16] ----
  const int m = lane & 15;
  if (m >= M) return;
  const float sa = sa_lds[m];
  const int nl = 4 * (lane >> 4);
  const int64_t n = n_base + nl;
  uint32_t y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (nl + r < rows_valid) {
      const float bb = HAS_BIAS ? bf16_to_f32(a.bias[n + r]) : 0.f;
      y[r] = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(acc[r], sa, a.w_scale[n + r], bb));
    } else {
      y[r] = 0;
    }
  }
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
      *reinterpret_cast<int4*>(dst) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nl + r < rows_valid) dst[r] = acc[r];
    }
  }
}

}  // namespace

hipError_t launch_small_m(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int64_t grid = (a.N + 63) / 64;
  const size_t lds = (size_t)16 * (size_t)xs_stride(a.K);
  const int vec_flags = epilogue_vec_flags(a);
  if (a.bias)
    hipLaunchKernelGGL(small_m_kernel<true>, dim3((unsigned)grid), dim3(256), lds, stream, x, ldx,
                       a, xq_out, a_scale_out, vec_flags);
  else
    hipLaunchKernelGGL(small_m_kernel<false>, dim3((unsigned)grid), dim3(256), lds, stream, x, ldx,
                       a, xq_out, a_scale_out, vec_flags);
  return hipGetLastError();
}

}  // namespace w8a8
