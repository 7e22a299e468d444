// Internal launch functions of libw8a8 (host side). Each enqueues kernels on
// `stream` and returns the launch status; arguments are validated by the
// C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Per-row symmetric int8 quantisation of R bf16 (f16: fp16) rows of length K.
hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t K, int64_t ldx,
                             int8_t* q, float* scale, hipStream_t stream, bool f16 = false);

struct GemmArgs {
  const int8_t* xq;        // [M, K]
  const float* a_scale;    // [M]
  const int8_t* wq;        // [N, K]
  const float* w_scale;    // [N]
  const uint16_t* bias;    // [N] or nullptr
  uint16_t* out;           // [M, ldo]
  int32_t* acc_debug;      // [M, N] or nullptr
  int64_t M, N, K, ldo;
  bool f16 = false;        // bias, out (and the small-M kernel's x) are fp16, not bf16
  // split-K: int32 partial sums [splits][M][N] (a workspace of at least
  // gemm_partial_bytes(M, N, K) bytes), or nullptr to compute every tile in
  // one workgroup
  int32_t* partial = nullptr;
};

// Bit 0: out rows allow 8-byte stores of four bf16 (out 8-byte aligned,
// ldo % 4 == 0, N % 4 == 0). Bit 1: acc_debug allows 16-byte stores
// (16-byte aligned, N % 4 == 0). Bit 2: out rows allow 16-byte stores of
// eight bf16 (out 16-byte aligned, ldo % 8 == 0, N % 8 == 0). Lanes own
// column groups that start at multiples of the store width, so these
// conditions make every vector store aligned and all-or-nothing at N.
inline int epilogue_vec_flags(const GemmArgs& a) {
  const uintptr_t ob = reinterpret_cast<uintptr_t>(a.out);
  const uintptr_t db = reinterpret_cast<uintptr_t>(a.acc_debug);
  int f = 0;
  if ((ob & 7) == 0 && (a.ldo & 3) == 0 && (a.N & 3) == 0) f |= 1;
  if ((db & 15) == 0 && (a.N & 3) == 0) f |= 2;
  if ((ob & 15) == 0 && (a.ldo & 7) == 0 && (a.N & 7) == 0) f |= 4;
  return f;
}

// Tile (BM x BN) the MFMA GEMM picks for a shape.
void gemm_pick_tile(int64_t M, int64_t N, int64_t K, int* bm, int* bn);

// int8 MFMA GEMM with the fused scale epilogue. With a.partial set and a
// shape whose large tiles leave most compute units idle, K is split in two
// and a second kernel adds the int32 partial sums (exactly) before the same
// epilogue.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// Bytes of partial sums launch_gemm uses for this shape on the current
// device (0: no split).
size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K);

// Small-M path: per-row activation quantisation on chip + weight-streaming
// MFMA product + epilogue, one kernel. Also writes xq/a_scale to xq_out /
// a_scale_out. Needs M <= 16 and K <= kSmallMMaxK, or M <= kSmallMWideRows
// and K <= kSmallMWideMaxK (the quantised rows are held in LDS).
constexpr int64_t kSmallMMaxK = 8192;
constexpr int64_t kSmallMWideRows = 32;
constexpr int64_t kSmallMWideMaxK = 4096;
hipError_t launch_small_m(const uint16_t* x, int64_t ldx, const GemmArgs& a,
                          int8_t* xq_out, float* a_scale_out, hipStream_t stream);

// compressed-tensors pack-quantized ingest: packed [N, ldp] int32 (uint8
// offset by 128, four to a word, little-endian) -> wq [N, K] int8, and scale_in
// [N] (kScaleF32 / kScaleBF16 / kScaleF16) -> w_scale [N] fp32. K % 16 == 0,
// ldp % 4 == 0, packed and wq 16-byte aligned.
constexpr int kScaleF32 = 0, kScaleBF16 = 1, kScaleF16 = 2;
hipError_t launch_unpack(const int32_t* packed, int64_t N, int64_t K, int64_t ldp, const void* scale_in,
                         int scale_dtype, int8_t* wq, float* w_scale, hipStream_t stream);

// W8A16 small-M linear: bf16 x [M, ldx] (M <= 16), int8 wq, fp32 w_scale,
// fp32 accumulation, bf16 out. a.xq / a.a_scale / a.acc_debug are unused.
// Needs w8a16_lds_bytes(M, K) <= kW8A16MaxLds bytes of LDS.
constexpr size_t kW8A16MaxLds = 128 * 1024;
size_t w8a16_lds_bytes(int64_t M, int64_t K);
hipError_t launch_w8a16(const uint16_t* x, int64_t ldx, const GemmArgs& a, hipStream_t stream);

}  // namespace w8a8
