// compressed-tensors pack-quantized ingest: int32-packed weights -> int8 [N, K]
// plus fp32 per-output-channel scales (gfx950).
//
// The pages' int8 weight-only checkpoint stores each weight as an unsigned byte
// offset by 128, four to a 32-bit word (Issue 5 probe, "Round one: int8 weight-only via
// compressed-tensors": the artifact is written with compressed-tensors'
// pack_to_int32). Element 4i+j of a row sits in bits 8j..8j+7 of word i
// (little-endian, the first element in the low byte), so the unpacked int8
// value is the stored byte minus 128, i.e. the byte with its top bit flipped.
// The per-channel scales arrive as fp32, bf16 or fp16 and leave as fp32
// (all three convert exactly).
//
// HBM-bound: 16-byte non-temporal loads (four words, sixteen weights) and
// 16-byte stores, four per thread in flight, grid-strided over the chunks;
// the scale conversion rides in the same launch.
#include <algorithm>

#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kUnroll = 4;   // chunks in flight per thread

__device__ __forceinline__ float scale_to_f32(const void* in, int dtype, int64_t i) {
  if (dtype == kScaleF32) return static_cast<const float*>(in)[i];
  if (dtype == kScaleBF16) return bf16_to_f32(static_cast<const uint16_t*>(in)[i]);
  return (float)static_cast<const _Float16*>(in)[i];
}

// One launch for both outputs: the scales (N values, grid-strided), then the
// weights. K % 16 == 0, ldp % 4 == 0 and 16-byte aligned rows: every chunk is
// four whole words on both sides. wq is [N, K] contiguous, so chunk i is at
// byte 16*i of it; the packed side is contiguous too unless ldp > K/4 (then
// the row comes from one division per chunk).
template <bool CONTIG>
__global__ __launch_bounds__(256) void unpack_kernel(const int32_t* __restrict__ packed, int64_t N,
                                                     int64_t K, int64_t ldp, int8_t* __restrict__ wq,
                                                     const void* __restrict__ scale_in, int scale_dtype,
                                                     float* __restrict__ w_scale) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * 256;
  for (int64_t i = tid; i < N; i += nthreads) w_scale[i] = scale_to_f32(scale_in, scale_dtype, i);

  const int64_t per_row = K / 16;                       // 16-byte chunks per row
  const int64_t total = N * per_row;
  const v4i flip = (v4i){(int)0x80808080, (int)0x80808080, (int)0x80808080, (int)0x80808080};
  auto src = [&](int64_t i) -> const v4i* {
    if constexpr (CONTIG) return reinterpret_cast<const v4i*>(packed + 4 * i);
    const int64_t row = i / per_row;
    return reinterpret_cast<const v4i*>(packed + row * ldp + 4 * (i - row * per_row));
  };
  for (int64_t base = tid; base < total; base += nthreads * kUnroll) {
    v4i v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * nthreads;
      if (i < total) v[u] = __builtin_nontemporal_load(src(i));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * nthreads;
      if (i < total) *reinterpret_cast<v4i*>(wq + 16 * i) = v[u] ^ flip;
    }
  }
}

}  // namespace

hipError_t launch_unpack(const int32_t* packed, int64_t N, int64_t K, int64_t ldp, const void* scale_in,
                         int scale_dtype, int8_t* wq, float* w_scale, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t chunks = N * (K / 16);
  const int64_t grid = std::max<int64_t>(
      1, std::min<int64_t>((chunks + 256 * kUnroll - 1) / (256 * kUnroll), 256 * 16));
  if (ldp * 4 == K)
    hipLaunchKernelGGL(unpack_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, packed, N, K, ldp,
                       wq, scale_in, scale_dtype, w_scale);
  else
    hipLaunchKernelGGL(unpack_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, packed, N, K,
                       ldp, wq, scale_in, scale_dtype, w_scale);
  return hipGetLastError();
}

}  // namespace w8a8
