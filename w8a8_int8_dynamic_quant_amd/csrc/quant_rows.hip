// Per-row symmetric int8 quantisation of bf16 rows (gfx950).
//
// Serves both the dynamic per-token activation quantisation and the
// load-time per-output-channel weight quantisation of the W8A8 int8-dynamic
// linear (Issue 5 probe, "Round two"; Int8 Quantization guide, "Overview").
//
// One wave64 per row, four rows per 256-thread workgroup. Each lane issues
// all of its 16-byte loads (8 bf16 each) for the row at once, through a
// buffer descriptor bounded at the row end, so chunks past K read as zero
// (which leaves amax unchanged) without any branch; a wave reads 1 KiB
// contiguous per instruction. The row stays in registers between the amax
// pass and the quantise pass (up to CHUNKS chunks per lane), so x is read
// from HBM exactly once. amax is an integer max over |x| bit patterns with a
// DPP butterfly across the wave. Output: 8 int8 per lane and chunk (8-byte
// buffer stores, 512 B contiguous per wave) and one fp32 scale per row.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr uint32_t kOOB = 0x7ffffff0u;   // an offset past every descriptor bound

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__device__ __forceinline__ void store8(uint2 q, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64((v2u){q.x, q.y}, r, off, 0, 0);
}

// Unsigned max over the 64 lanes of the wave (DPP within rows of 16, then
// row broadcasts), returned as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false)); // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false)); // row_ror 8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast 15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false)); // row_bcast 31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int CHUNKS>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  // wave-uniform row (readfirstlane keeps the row's buffer descriptor scalar)
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= R) return;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * ldx, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rq = row_rsrc(q + row * K, (uint32_t)K);

  uint4 v[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) v[c] = load16(rx, (uint32_t)(lane + 64 * c) * 16u);
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) amax = absmax_bits8(v[c], amax);
  amax = wave_max_dpp(amax);
  const float s = row_scale(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;  // subnormal s
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const uint32_t idx = (uint32_t)(lane + 64 * c);
    store8(quant8(v[c], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
  }
  if (lane == 0) scale[row] = s;
}

// Rows longer than the register-resident limit: amax pass, then a second
// pass that re-reads the row (from L2 for the row lengths that get here).
__global__ __launch_bounds__(256) void quant_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= R) return;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * ldx, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rq = row_rsrc(q + row * K, (uint32_t)K);
  uint32_t amax = 0;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) amax = absmax_bits8(v[u], amax);
  }
  amax = wave_max_dpp(amax);
  const float s = row_scale(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      store8(quant8(v[u], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
    }
  }
  if (lane == 0) scale[row] = s;
}

}  // namespace

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
