// compressed-tensors pack-quantized ingest: int32-packed weights -> int8 [N, K]
// plus fp32 per-output-channel scales (gfx950).
//
// The pages' int8 weight-only checkpoint stores each weight as uint8 biased by
// 128, four per int32 (Issue 5 probe, "Round one: int8 weight-only via
// compressed-tensors": the artifact is written with compressed-tensors'
// pack_to_int32). Element 4i+j of a row sits in bits 8j..8j+7 of word i
// (little-endian, the first element in the low byte), so the unpacked int8
// value is the stored byte minus 128, i.e. the byte with its top bit flipped.
// The per-channel scales arrive as fp32, bf16 or fp16 and leave as fp32
// (all three convert exactly).
//
// HBM-bound: one 16-byte load (four words, sixteen weights) and one 16-byte
// store per thread per step, grid-strided over rows x 16-byte chunks.
#include <algorithm>

#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

// K % 16 == 0, ldp % 4 == 0 and 16-byte aligned rows: every chunk is four
// whole words on both sides.
__global__ __launch_bounds__(256) void unpack_kernel(const int32_t* __restrict__ packed, int64_t N,
                                                     int64_t K, int64_t ldp, int8_t* __restrict__ wq) {
  const int64_t per_row = K / 16;                       // 16-byte chunks per row
  const int64_t total = N * per_row;
  const v4i flip = (v4i){(int)0x80808080, (int)0x80808080, (int)0x80808080, (int)0x80808080};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row, c = i - row * per_row;
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(packed + row * ldp + 4 * c));
    *reinterpret_cast<v4i*>(wq + row * K + 16 * c) = v ^ flip;
  }
}

__global__ __launch_bounds__(256) void scales_kernel(const void* __restrict__ in, int dtype, int64_t N,
                                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  float s;
  if (dtype == kScaleF32) {
    s = static_cast<const float*>(in)[i];
  } else if (dtype == kScaleBF16) {
    s = bf16_to_f32(static_cast<const uint16_t*>(in)[i]);
  } else {
    s = (float)static_cast<const _Float16*>(in)[i];
  }
  out[i] = s;
}

}  // namespace

hipError_t launch_unpack(const int32_t* packed, int64_t N, int64_t K, int64_t ldp, const void* scale_in,
                         int scale_dtype, int8_t* wq, float* w_scale, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t chunks = N * (K / 16);
  const int64_t grid = std::min<int64_t>((chunks + 255) / 256, 256 * 16);
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, packed, N, K, ldp, wq);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL(scales_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, scale_in,
                     scale_dtype, N, w_scale);
  return hipGetLastError();
}

}  // namespace w8a8
