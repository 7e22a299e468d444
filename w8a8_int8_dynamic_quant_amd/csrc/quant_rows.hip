// Per-row symmetric int8 quantisation of bf16 or fp16 rows (gfx950).
//
// Serves both the dynamic per-token activation quantisation and the
// load-time per-output-channel weight quantisation of the W8A8 int8-dynamic
// linear (Issue 5 probe, "Round two"; Int8 Quantization guide, "Overview").
//
// Rows of up to 4096 elements: one or two waves per row (two from 1536
// elements on, sharing the row's amax through LDS, so each wave's compute
// after its loads land is half as long). Rows of up to 32768 elements: a
// workgroup of 4 waves per row, thread t holding the row's 16-byte chunks t,
// t+256, ... (8 values each; 4 KiB contiguous per load instruction of the
// workgroup), the four wave maxima meeting in LDS. Either way every chunk of
// a row is requested at once and the whole matrix is launched at once (a
// persistent grid walking rows with the next row prefetched measured slower:
// 34.3 against 29.8 us for 4352 x 12288). Loads go through a buffer
// descriptor bounded at the row end, so chunks past K read as zero (which
// leaves amax unchanged) without any branch, and are non-temporal (x is read
// once). amax is an integer max over |x| bit patterns with a DPP butterfly
// within each wave. Output: 8 int8 per chunk (8-byte stores) and one fp32
// scale per row. Longer rows use a two-pass kernel (amax pass, then a
// quantise pass re-reading the row).
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

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


template <int CHT, bool F16>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t wmax[4];             // per-wave amax
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const int64_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row * ldx, (uint32_t)K * 2u);
  uint4 v[CHT];
#pragma unroll
  for (int u = 0; u < CHT; ++u) v[u] = load16_nt(rx, (uint32_t)(tid + 256 * u) * 16u);
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < CHT; ++u) amax = absmax_bits8(v[u], amax);
  amax = wave_max_dpp(amax);
  if ((tid & 63) == 0) wmax[wave] = amax;
  lds_barrier();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;  // subnormal s
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row * K, (uint32_t)K);
#pragma unroll
  for (int u = 0; u < CHT; ++u) {
    const uint32_t idx = (uint32_t)(tid + 256 * u);
    store8(quant8<F16>(v[u], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
  }
  if (tid == 0) scale[row] = s;
}

// Short rows: P waves per row (P = 1 or 2), 4/P rows per workgroup; wave
// part h of a row holds chunks lane + 64*(c + CHUNKS*h), c < CHUNKS, all
// requested at once and kept in registers between the amax and the quantise
// step; all rows are in flight together. With P = 2 the two waves exchange
// their amax through LDS.
template <int CHUNKS, int P, bool F16>
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  static_assert(P == 1 || P == 2, "one or two waves per row");
  __shared__ uint32_t part_max[4];
  const int lane = threadIdx.x & 63;
  // wave-uniform row (readfirstlane keeps the row's buffer descriptor scalar)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % P;
  const int64_t row = (int64_t)blockIdx.x * (4 / P) + wave / P;
  const bool valid = row < R;
  if (P == 1 && !valid) return;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  // past the last row the descriptor is empty: every load reads zero
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(x + (valid ? row : 0) * ldx, valid ? (uint32_t)K * 2u : 0u);
  uint4 v[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c)
    v[c] = load16_nt(rx, (uint32_t)(lane + 64 * (c + CHUNKS * part)) * 16u);
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) amax = absmax_bits8(v[c], amax);
  amax = wave_max_dpp(amax);
  if constexpr (P == 2) {
    if (lane == 0) part_max[wave] = amax;
    lds_barrier();
    amax = max(part_max[wave & 2], part_max[(wave & 2) + 1]);
    if (!valid) return;
  }
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row * K, (uint32_t)K);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;  // subnormal s
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const uint32_t idx = (uint32_t)(lane + 64 * (c + CHUNKS * part));
    store8(quant8<F16>(v[c], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
  }
  if (lane == 0 && part == 0) scale[row] = s;
}

// Rows longer than the register-resident limit: one wave per row, an amax
// pass, then a second pass that re-reads the row (from L2 for the row
// lengths that get here).
template <bool F16>
__global__ __launch_bounds__(256) void quant_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= R) return;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row * ldx, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row * K, (uint32_t)K);
  uint32_t amax = 0;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) amax = absmax_bits8(v[u], amax);
  }
  amax = wave_max_dpp(amax);
  const float s = row_scale<F16>(amax);
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
      store8(quant8<F16>(v[u], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
    }
  }
  if (lane == 0) scale[row] = s;
}

template <int C, bool F16>
hipError_t launch_cht(const uint16_t* x, int64_t R, int64_t K, int64_t ldx, int8_t* q, float* scale,
                      hipStream_t stream) {
  hipLaunchKernelGGL((quant_rows_kernel<C, F16>), dim3((unsigned)R), dim3(256), 0, stream, x, R, K,
                     ldx, q, scale);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_quant_rows_t(const uint16_t* x, int64_t R, int64_t K, int64_t ldx,
                               int8_t* q, float* scale, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int64_t nchunks = K >> 3;
  const int64_t per_lane = (nchunks + 63) / 64;
  if (per_lane <= 8) {                    // K <= 4096: one or two waves per row
    const dim3 block(256);
#define W8A8_QW(C, P)                                                                   \
    hipLaunchKernelGGL((quant_rows_wave_kernel<C, P, F16>),                             \
                       dim3((unsigned)((R + 4 / P - 1) / (4 / P))), block, 0, stream, x, R, \
                       K, ldx, q, scale);                                               \
    return hipGetLastError();
    if (per_lane <= 1) { W8A8_QW(1, 1) }
    if (per_lane <= 2) { W8A8_QW(2, 1) }
    if (per_lane <= 4) { W8A8_QW(2, 2) }
    if (per_lane <= 6) { W8A8_QW(3, 2) }
    W8A8_QW(4, 2)
#undef W8A8_QW
  }
  const int64_t per_thread = (nchunks + 255) / 256;
  if (per_thread <= 4) return launch_cht<4, F16>(x, R, K, ldx, q, scale, stream);
  if (per_thread <= 6) return launch_cht<6, F16>(x, R, K, ldx, q, scale, stream);
  if (per_thread <= 8) return launch_cht<8, F16>(x, R, K, ldx, q, scale, stream);
  if (per_thread <= 12) return launch_cht<12, F16>(x, R, K, ldx, q, scale, stream);
  if (per_thread <= 16) return launch_cht<16, F16>(x, R, K, ldx, q, scale, stream);
  hipLaunchKernelGGL(quant_rows_long_kernel<F16>, dim3((unsigned)((R + 3) / 4)), dim3(256), 0,
                     stream, x, R, K, ldx, q, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t K, int64_t ldx, int8_t* q,
                             float* scale, hipStream_t stream, bool f16) {
  return f16 ? launch_quant_rows_t<true>(x, R, K, ldx, q, scale, stream)
             : launch_quant_rows_t<false>(x, R, K, ldx, q, scale, stream);
}

}  // namespace w8a8
