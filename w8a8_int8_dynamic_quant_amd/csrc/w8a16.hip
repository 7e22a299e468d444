// W8A16 linear for M <= 16: int8 weights with fp32 per-output-channel scales,
// bf16 (or fp16) activations used as they are (no activation quantisation)
// (gfx950).
//
// The int8 weight-only scheme of the Issue 5 probe ("Round one: int8
// weight-only via compressed-tensors"), for the small-M layers that stream
// their weight once from HBM:
//   acc[m,n] = sum_k fp32(x[m,k]) * wq[n,k]      (fp32 accumulation)
//   y[m,n]   = bf16(fl32(acc * s_w[n]) + bias[n])
// Every bf16 x int8 product is exact in fp32; the accumulation order is the
// MFMA's.
//
// Workgroups of W waves (4..12, one workgroup per CU when the weight allows;
// see row_groups.h), each wave 8 weight rows over all of K in 128-byte
// windows, as the W8A8 small-M kernel:
//  1. the M activation rows are copied into LDS as bf16 by LDS-DMA
//     (buffer_load ... lds) before any weight window is requested; chunks
//     past K read as zero through the descriptor bound, so the padded tail
//     of each row (up to its last 128-element window) is zero, never NaN
//     garbage meeting a zero weight;
//  2. the wave requests up to kD windows at once (lane l: row l%8, 16-byte
//     chunk l/8 = 16 int8), widens each to bf16 in registers (exact:
//     |q| <= 128 has at most 8 significant bits) and runs two
//     v_mfma_f32_16x16x32_bf16 per window per 8 tokens, reading A-row i as
//     weight row i%8 at chunk parity i/8 (B built the same way from LDS), so
//     D[n][t] + D[n+8][t+8] is the dot product of row n and token t;
//  3. epilogue in fp32: (acc * s_w) + bias, bf16 round to nearest even.
#include "row_groups.h"
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kD = 24;                   // 128-byte windows in flight per wave

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Bytes per LDS activation row: K bf16 rounded up to whole 128-element
// windows, plus room for the per-token shift of w8a16_row_offset.
__host__ __device__ inline int w8a16_row_bytes(int64_t K) { return (int)((K + 127) / 128 + 1) * 256; }

// LDS offset of token t's row. The B read of a quarter-wave takes tokens
// 0..7 at 16-byte chunk parities 0/1; shifting row t by 16*(4*(t%4) + (t/4)%2)
// bytes puts those 16 reads in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int w8a16_row_offset(int t, int row_bytes) {
  return t * row_bytes + 16 * (4 * (t & 3) + ((t >> 2) & 1));
}

// Eight signed bytes (two words) -> eight bf16, exactly.
__device__ __forceinline__ v8bf widen8(uint32_t lo, uint32_t hi) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? lo : hi;
    const int sh = 16 * (i & 1);
    const float f0 = (float)(int)(signed char)(w >> sh);
    const float f1 = (float)(int)(signed char)(w >> (sh + 8));
    // high halves of the two floats: bytes 2,3 of f0 then bytes 2,3 of f1
    o[i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, (v4u){o[0], o[1], o[2], o[3]});
}

// Eight signed bytes (two words) -> eight fp16, exactly, with one byte
// permute per pair: the biased byte u = q + 128 (q with its top bit flipped)
// under the byte 0x64 is the fp16 value 1024 + u, and one packed fp16
// subtraction of 1152 leaves q (every step exact: integers below 2048).
__device__ __forceinline__ v8h widen8_f16(uint32_t lo, uint32_t hi) {
  const uint32_t ulo = lo ^ 0x80808080u, uhi = hi ^ 0x80808080u;
  // selector bytes 0-3 pick from the second operand, 4-7 from the first
  const v4u o = {__builtin_amdgcn_perm(0x64646464u, ulo, 0x04010400u),
                 __builtin_amdgcn_perm(0x64646464u, ulo, 0x04030402u),
                 __builtin_amdgcn_perm(0x64646464u, uhi, 0x04010400u),
                 __builtin_amdgcn_perm(0x64646464u, uhi, 0x04030402u)};
  const _Float16 off = (_Float16)1152.0f;
  return __builtin_bit_cast(v8h, o) - (v8h){off, off, off, off, off, off, off, off};
}

template <bool HAS_BIAS, bool TWO, bool LONG, bool F16>
__global__ __launch_bounds__(64 * kMaxWaves) void w8a16_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                    GemmArgs a, int vec_flags) {
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = blockDim.x >> 6;
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int row_bytes = w8a16_row_bytes(K);
  const int nwin = (int)((K + 127) / 128);
  const int64_t n_base = ((int64_t)blockIdx.x * W + wave) * 8;
  const int rows_valid = (int)max<int64_t>(0, min<int64_t>(8, N - n_base));
  // epilogue scale and bias (row n_base + lane % 8), requested before anything else
  float sw1, bb1;
  load_row_scale<HAS_BIAS, F16>(a.w_scale, a.bias, n_base, rows_valid, lane, sw1, bb1);

  // ---- 1. activation rows into LDS (LDS-DMA: lane l of an instruction
  // writes the 16 bytes at LDS base + 16*l) ----
  // A row takes nwin*256 bytes; lanes past that are masked off so that the
  // last instruction of a row never writes into the next row's bytes.
  const int row_used = nwin * 256;
  const int chunks = (row_used + 1023) / 1024;
  for (int m = wave; m < M; m += W) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, (uint32_t)K * 2u);
    int8_t* dst = xs + w8a16_row_offset(m, row_bytes);
    for (int c = 0; c < chunks; ++c)
      if (1024 * c + 16 * lane < row_used)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst + 1024 * c, 16, (uint32_t)(1024 * c + 16 * lane),
                                                 0, 0, 0);
  }
  // The rows land before any weight window is requested: with the windows
  // requested right behind the copies, the other waves' weight requests
  // delayed the copies that every wave then waits for (M = 1: 15.2 against
  // 13.3 us per call).
  __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): this wave's rows have landed
  __syncthreads();                         // ... and every other wave's
  if (rows_valid == 0) return;

  // ---- 2. weight windows ----
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
#pragma unroll
  for (int d = 0; d < kD; ++d) buf[d] = wload(d);
  __builtin_amdgcn_sched_barrier(0);       // all requests out before the first use

  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  const int8_t* xb0 = xs + w8a16_row_offset(lane & 7, row_bytes) + 32 * chunk;
  const int8_t* xb1 = xs + w8a16_row_offset(8 + (lane & 7), row_bytes) + 32 * chunk;
  // window w: widen, then per 8-element half e one MFMA per token block;
  // windows past the end multiply zero weights, so the LDS read is kept
  // inside the row (its last window)
  auto window = [&](int w, const v4i& wv) {
    const int wc = min(w, nwin - 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if constexpr (F16) {
        const v8h A = widen8_f16((uint32_t)wv[2 * e], (uint32_t)wv[2 * e + 1]);
        const v8h B0 = *reinterpret_cast<const v8h*>(xb0 + 256 * wc + 16 * e);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B0, acc0, 0, 0, 0);
        if constexpr (TWO) {
          const v8h B1 = *reinterpret_cast<const v8h*>(xb1 + 256 * wc + 16 * e);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B1, acc1, 0, 0, 0);
        }
      } else {
        const v8bf A = widen8((uint32_t)wv[2 * e], (uint32_t)wv[2 * e + 1]);
        const v8bf B0 = *reinterpret_cast<const v8bf*>(xb0 + 256 * wc + 16 * e);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc0, 0, 0, 0);
        if constexpr (TWO) {
          const v8bf B1 = *reinterpret_cast<const v8bf*>(xb1 + 256 * wc + 16 * e);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc1, 0, 0, 0);
        }
      }
    }
  };
  if constexpr (!LONG) {
#pragma unroll
    for (int d = 0; d < kD; ++d) window(d, buf[d]);
  } else {
    for (int base = 0; base < nwin; base += kD) {
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        window(base + d, buf[d]);
        buf[d] = wload(base + d + kD);
      }
    }
  }

  // ---- 3. epilogue ----
  // D[i][j] sits in lane 16*(i/4) + j, element i%4. Row n < 8 at token t < 8
  // is D[n][t] + D[n+8][t+8], the second term 40 lanes up; lanes 0-7 and
  // 16-23 then hold rows nl..nl+3 (nl = 4*(lane/16)) of token lane%8.
  // (Elements are copied out by value first: a bit cast taken directly of a
  // vector element reads the vector's first element.)
  const int src = ((lane + 40) & 63) * 4;
  float s0[4], s1[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float c0 = acc0[r], c1 = acc1[r];
    s0[r] = c0 + __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(c0)));
    s1[r] = TWO ? c1 + __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(c1))) : 0.f;
  }
  float sw[4], bb[4];
  gather4(sw1, 4 * ((lane >> 4) & 1), sw);
  gather4(bb1, 4 * ((lane >> 4) & 1), bb);
  if ((lane & 8) != 0 || lane >= 32) return;
  const int nl = 4 * (lane >> 4);
  const int64_t n = n_base + nl;
#pragma unroll
  for (int blk = 0; blk < (TWO ? 2 : 1); ++blk) {
    const int m = 8 * blk + (lane & 7);
    if (m >= M) continue;
    const float* c = blk ? s1 : s0;
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma clang fp contract(off)
      float t = c[r] * sw[r];
      if (HAS_BIAS) t = t + bb[r];
      y[r] = f32_to_half_rne<F16>(t);
    }
    uint16_t* o = a.out + (int64_t)m * a.ldo + n;
    if (nl + 3 < rows_valid && (vec_flags & 1)) {
      *reinterpret_cast<uint2*>(o) = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nl + r < rows_valid) o[r] = (uint16_t)y[r];
    }
  }
}

template <bool HAS_BIAS, bool TWO, bool F16>
hipError_t launch_w8a16_variant(const uint16_t* x, int64_t ldx, const GemmArgs& a, hipStream_t stream) {
  const RowGroupGrid g = row_group_grid(a.N);
  const dim3 grid(g.blocks), block(64 * g.waves);
  const size_t lds = (size_t)(TWO ? 16 : 8) * (size_t)w8a16_row_bytes(a.K);
  const int vf = epilogue_vec_flags(a);
  if (a.K > 128 * kD)
    hipLaunchKernelGGL((w8a16_kernel<HAS_BIAS, TWO, true, F16>), grid, block, lds, stream, x, ldx, a,
                       vf);
  else
    hipLaunchKernelGGL((w8a16_kernel<HAS_BIAS, TWO, false, F16>), grid, block, lds, stream, x, ldx,
                       a, vf);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_w8a16_dtype(const uint16_t* x, int64_t ldx, const GemmArgs& a,
                              hipStream_t stream) {
  if (a.bias)
    return a.M > 8 ? launch_w8a16_variant<true, true, F16>(x, ldx, a, stream)
                   : launch_w8a16_variant<true, false, F16>(x, ldx, a, stream);
  return a.M > 8 ? launch_w8a16_variant<false, true, F16>(x, ldx, a, stream)
                 : launch_w8a16_variant<false, false, F16>(x, ldx, a, stream);
}

}  // namespace

size_t w8a16_lds_bytes(int64_t M, int64_t K) {
  return (size_t)(M > 8 ? 16 : 8) * (size_t)w8a16_row_bytes(K);
}

hipError_t launch_w8a16(const uint16_t* x, int64_t ldx, const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  return a.f16 ? launch_w8a16_dtype<true>(x, ldx, a, stream)
               : launch_w8a16_dtype<false>(x, ldx, a, stream);
}

}  // namespace w8a8
