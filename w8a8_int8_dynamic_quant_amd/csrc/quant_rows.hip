// Per-row symmetric int8 quantisation of bf16 rows (gfx950).
//
// Serves both the dynamic per-token activation quantisation and the
// load-time per-output-channel weight quantisation of the W8A8 int8-dynamic
// linear (Issue 5 probe, "Round two"; Int8 Quantization guide, "Overview").
//
// One wave64 per row, four rows per 256-thread workgroup. Each lane loads
// 16-byte chunks (8 bf16) so a wave reads 1 KiB contiguous per instruction;
// the row stays in registers between the amax pass and the quantise pass
// (up to CHUNKS chunks per lane), so x is read from HBM exactly once.
// amax is an integer max over |x| bit patterns followed by a butterfly
// reduction across the wave. Output: 8 int8 per lane per chunk (8-byte
// stores, 512 B contiguous per wave) and one fp32 scale per row.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

template <int CHUNKS>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
  uint2* dst = reinterpret_cast<uint2*>(q + row * K);
  const int nchunks = (int)(K >> 3);

  uint4 v[CHUNKS];
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) {
      v[c] = load_nt16(src + idx);
      amax = absmax_bits8(v[c], amax);
    }
  }
  amax = wave_max_u32(amax);
  const float s = row_scale(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;  // subnormal s
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) dst[idx] = quant8(v[c], s, r, zero, exact_div);
  }
  if (lane == 0) scale[row] = s;
}

// Rows longer than the register-resident limit: amax pass, then a second
// pass that re-reads the row (from L2 for the row lengths that get here).
__global__ __launch_bounds__(256) void quant_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
  uint2* dst = reinterpret_cast<uint2*>(q + row * K);
  const int64_t nchunks = K >> 3;
  uint32_t amax = 0;
  for (int64_t idx = lane; idx < nchunks; idx += 64) amax = absmax_bits8(src[idx], amax);
  amax = wave_max_u32(amax);
  const float s = row_scale(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  for (int64_t idx = lane; idx < nchunks; idx += 64) dst[idx] = quant8(src[idx], s, r, zero, exact_div);
  if (lane == 0) scale[row] = s;
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t K, int64_t ldx,
                             int8_t* q, float* scale, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int64_t nchunks = K >> 3;
  const int64_t per_lane = (nchunks + 63) / 64;
  dim3 grid((unsigned)((R + 3) / 4)), block(256);
#define W8A8_QR(C)                                                                     \
  if (per_lane <= C) {                                                                 \
    hipLaunchKernelGGL(quant_rows_kernel<C>, grid, block, 0, stream, x, R, K, ldx, q, scale); \
    return hipGetLastError();                                                          \
  }
  W8A8_QR(1)
  W8A8_QR(2)
  W8A8_QR(4)
  W8A8_QR(6)
  W8A8_QR(8)
  W8A8_QR(12)
  W8A8_QR(16)
  W8A8_QR(24)
  W8A8_QR(32)
#undef W8A8_QR
  hipLaunchKernelGGL(quant_rows_long_kernel, grid, block, 0, stream, x, R, K, ldx, q, scale);
  return hipGetLastError();
}

}  // namespace w8a8
