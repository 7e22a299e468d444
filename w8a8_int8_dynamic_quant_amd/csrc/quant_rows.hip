// Per-row symmetric int8 quantisation of bf16 or fp16 rows (gfx950).
//
// Serves both the dynamic per-token activation quantisation and the
// load-time per-output-channel weight quantisation of the W8A8 int8-dynamic
// linear (Issue 5 probe, "Round two"; Int8 Quantization guide, "Overview").
//
// Rows of up to 4096 elements: one to four waves per row (two from 1025
// elements on, three from 2049, four from 3073; rows of 2049-3072 elements
// take two waves when there are more than 2048 rows), sharing the row's amax
// through LDS, so each wave's compute after its loads land is short. Rows
// of up to 32768 elements: a workgroup of NW = 8 waves per row (4 for rows
// of up to 8192 elements when there are more than 2048 rows), thread t
// holding the row's 16-byte chunks t, t + 64 NW, ... (8 values each; 64 NW
// x 16 bytes contiguous per load instruction of the workgroup), the wave
// maxima meeting in LDS. Either way every chunk of
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

template <int CHT, int NW, bool F16>
__global__ __launch_bounds__(64 * NW) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t wmax[NW];            // per-wave amax
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const int64_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row * ldx, (uint32_t)K * 2u);
  uint4 v[CHT];
#pragma unroll
  for (int u = 0; u < CHT; ++u) v[u] = load16_nt(rx, (uint32_t)(tid + 64 * NW * u) * 16u);
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < CHT; ++u) amax = absmax_bits8(v[u], amax);
  amax = wave_max_u32(amax);
  if ((tid & 63) == 0) wmax[wave] = amax;
  lds_barrier();
  amax = wmax[0];
#pragma unroll
  for (int h = 1; h < NW; ++h) amax = max(amax, wmax[h]);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;  // subnormal s
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row * K, (uint32_t)K);
#pragma unroll
  for (int u = 0; u < CHT; ++u) {
    const uint32_t idx = (uint32_t)(tid + 64 * NW * u);
    store8(quant8<F16>(v[u], s, r, zero, exact_div), rq, idx < nchunks ? idx * 8u : kOOB);
  }
  if (tid == 0) scale[row] = s;
}

// Short rows: P waves per row (P = 1 to 4), 4/P rows per workgroup (two
// for P = 3); wave part h of a row holds chunks lane + 64*(c + CHUNKS*h),
// c < CHUNKS, all requested at once and kept in registers between the amax
// and the quantise step; all rows are in flight together. With P > 1 the
// waves of a row exchange their amax through LDS.
template <int P>
constexpr int qw_rows_per_block() { return P == 3 ? 2 : 4 / P; }

template <int CHUNKS, int P, bool F16>
__global__ __launch_bounds__(64 * P * qw_rows_per_block<P>()) void quant_rows_wave_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int64_t ldx,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  static_assert(P >= 1 && P <= 4, "waves per row");
  constexpr int RPB = qw_rows_per_block<P>();
  __shared__ uint32_t part_max[RPB * P];
  const int lane = threadIdx.x & 63;
  // wave-uniform row (readfirstlane keeps the row's buffer descriptor scalar)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % P;
  const int64_t row = (int64_t)blockIdx.x * RPB + wave / P;
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
  amax = wave_max_u32(amax);
  if constexpr (P > 1) {
    if (lane == 0) part_max[wave] = amax;
    lds_barrier();
    const int base = wave - part;
    amax = part_max[base];
#pragma unroll
    for (int h = 1; h < P; ++h) amax = max(amax, part_max[base + h]);
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
  amax = wave_max_u32(amax);
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

template <int C, int NW, bool F16>
hipError_t launch_cht(const uint16_t* x, int64_t R, int64_t K, int64_t ldx, int8_t* q, float* scale,
                      hipStream_t stream) {
  hipLaunchKernelGGL((quant_rows_kernel<C, NW, F16>), dim3((unsigned)R), dim3(64 * NW), 0, stream, x,
                     R, K, ldx, q, scale);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_quant_rows_t(const uint16_t* x, int64_t R, int64_t K, int64_t ldx,
                               int8_t* q, float* scale, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int64_t nchunks = K >> 3;
  const int64_t per_lane = (nchunks + 63) / 64;
  if (per_lane <= 8) {                    // K <= 4096: one to four waves per row
#define W8A8_QW(C, P)                                                                   \
    hipLaunchKernelGGL((quant_rows_wave_kernel<C, P, F16>),                             \
                       dim3((unsigned)((R + qw_rows_per_block<P>() - 1) / qw_rows_per_block<P>())), \
                       dim3(64 * P * qw_rows_per_block<P>()), 0, stream, x, R, K, ldx, q, scale); \
    return hipGetLastError();
    // three and four waves per row with two chunks a lane, rather than two
    // waves with three or four: per call, same bits, 64 / 512 / 1024 / 4352
    // rows of 4096 elements 3.6 / 4.2 / 5.2 / 11.5 us against 5.1 / 5.6 /
    // 6.5 / 12.4; of 3072 elements, 64 / 512 / 1024 / 2048 rows 3.6 / 4.0 /
    // 5.0 / 6.3 against 4.1 / 4.7 / 5.4 / 6.9, while 4352 rows measured the
    // same either way (10.0-10.3 us), so more rows than 2048 keep two waves
    if (per_lane <= 1) { W8A8_QW(1, 1) }
    if (per_lane <= 2) { W8A8_QW(2, 1) }
    if (per_lane <= 4) { W8A8_QW(2, 2) }
    if (per_lane <= 6) {
      if (R <= 2048) { W8A8_QW(2, 3) }
      W8A8_QW(3, 2)
    }
    W8A8_QW(2, 4)
#undef W8A8_QW
  }
  // eight waves per row rather than four (half the chunks a thread): per
  // call, same bits, 64 / 1024 / 4352 rows of 12288 elements 4.5 / 9.7 /
  // 26.9 us against 5.9 / 11.0 / 27.8; of 24576 elements 7.7 / 16.2 /
  // 52.1 against 11.2 / 19.4 / 54.4; of 8192 elements 4.2 / 7.4 against
  // 4.8 / 8.3 at 64 / 1024 rows, but 19.7 against 19.3 at 4352 rows, so
  // rows of up to 8192 elements keep four waves beyond 2048 rows
  const int64_t per8 = (nchunks + 511) / 512;     // chunks per thread of eight waves
  if (per8 <= 2 && R > 2048) return launch_cht<4, 4, F16>(x, R, K, ldx, q, scale, stream);
  if (per8 <= 2) return launch_cht<2, 8, F16>(x, R, K, ldx, q, scale, stream);
  if (per8 <= 3) return launch_cht<3, 8, F16>(x, R, K, ldx, q, scale, stream);
  if (per8 <= 4) return launch_cht<4, 8, F16>(x, R, K, ldx, q, scale, stream);
  if (per8 <= 6) return launch_cht<6, 8, F16>(x, R, K, ldx, q, scale, stream);
  if (per8 <= 8) return launch_cht<8, 8, F16>(x, R, K, ldx, q, scale, stream);
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
