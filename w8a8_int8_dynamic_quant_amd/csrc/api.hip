// C ABI of libw8a8 (declared in include/w8a8.h): argument validation, path
// dispatch and kernel launches on the caller's stream. Nothing is allocated
// and nothing is kept between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/w8a8.h"
#include "producers.h"
#include "w8a8_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_k(int64_t K) {
  if (K < 0) return W8A8_ERR_INVALID_ARG;
  if (K < 16 || (K % 16) != 0 || K > W8A8_K_MAX) return W8A8_ERR_UNSUPPORTED;
  return W8A8_OK;
}

int check_bf16_ld(int64_t ld, int64_t K) {
  if (ld < K) return W8A8_ERR_INVALID_ARG;
  if (ld % 8 != 0) return W8A8_ERR_UNSUPPORTED;
  return W8A8_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return W8A8_OK;
  g_last_hip_error = (int)e;
  return W8A8_ERR_HIP;
}

int quant_common(const uint16_t* x, int64_t R, int64_t K, int64_t ld, int8_t* q, float* scale,
                 void* stream, bool f16) {
  if (R < 0) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(K)) return s;
  if (int s = check_bf16_ld(ld, K)) return s;
  if (R == 0) return W8A8_OK;
  if (!x || !q || !scale) return W8A8_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return W8A8_ERR_MISALIGNED;
  return hip_status(w8a8::launch_quant_rows(x, R, K, ld, q, scale, (hipStream_t)stream, f16));
}

// Checks shared by the two GEMM entry points (everything but x / xq).
int check_gemm(int64_t M, int64_t K, int64_t N, const int8_t* wq, const float* w_scale,
               const uint16_t* bias, const uint16_t* out, int64_t ldo, const int32_t* acc_debug) {
  if (M < 0 || N < 1) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(K)) return s;
  if (ldo < N) return W8A8_ERR_INVALID_ARG;
  // a 256-row output tile (and the debug accumulators, row stride N) must be
  // addressable with 32-bit byte offsets
  if (ldo > W8A8_LDO_MAX || (acc_debug && N > W8A8_LDO_MAX / 2)) return W8A8_ERR_UNSUPPORTED;
  if (M == 0) return W8A8_OK;
  if (!wq || !w_scale || !out) return W8A8_ERR_INVALID_ARG;
  if (!aligned(wq, 16) || !aligned(w_scale, 4) || !aligned(out, 4)) return W8A8_ERR_MISALIGNED;
  if (bias && !aligned(bias, 2)) return W8A8_ERR_MISALIGNED;
  if (acc_debug && !aligned(acc_debug, 4)) return W8A8_ERR_MISALIGNED;
  return W8A8_OK;
}

bool small_m_path(int64_t M, int64_t K) {
  static_assert(W8A8_SMALL_M_WIDE == w8a8::kSmallMWideRows, "small-M row limits");
  return M >= 1 && ((M <= W8A8_SMALL_M && K <= w8a8::kSmallMMaxK) ||
                    (M <= W8A8_SMALL_M_WIDE && K <= w8a8::kSmallMWideMaxK));
}

int scaled_mm_common(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                     const int8_t* wq, const float* w_scale, int64_t N, const uint16_t* bias,
                     uint16_t* out, int64_t ldo, int32_t* acc_debug, void* stream, bool f16) {
  if (int s = check_gemm(M, K, N, wq, w_scale, bias, out, ldo, acc_debug)) return s;
  if (M == 0) return W8A8_OK;
  if (!xq || !a_scale) return W8A8_ERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(a_scale, 4)) return W8A8_ERR_MISALIGNED;
  w8a8::GemmArgs g{xq, a_scale, wq, w_scale, bias, out, acc_debug, M, N, K, ldo, f16};
  return hip_status(w8a8::launch_gemm(g, (hipStream_t)stream));
}

int linear_common(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                  const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out,
                  int64_t ldo, void* workspace, size_t workspace_bytes, int32_t* acc_debug,
                  void* stream, bool f16) {
  if (int s = check_gemm(M, K, N, wq, w_scale, bias, out, ldo, acc_debug)) return s;
  if (int s = check_bf16_ld(ldx, K)) return s;
  if (M == 0) return W8A8_OK;
  if (!x) return W8A8_ERR_INVALID_ARG;
  if (!aligned(x, 16)) return W8A8_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < w8a8_linear_workspace_bytes(M, K, N))
    return W8A8_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return W8A8_ERR_MISALIGNED;
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* a_scale = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            W8A8_ALIGN256((size_t)M * (size_t)K));
  hipStream_t st = (hipStream_t)stream;
  w8a8::GemmArgs g{xq, a_scale, wq, w_scale, bias, out, acc_debug, M, N, K, ldo, f16};
  if (small_m_path(M, K)) return hip_status(w8a8::launch_small_m(x, ldx, g, xq, a_scale, st));
  if (w8a8::gemm_partial_bytes(M, N, K) > 0)       // split-K partial sums follow a_scale
    g.partial = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                           W8A8_ALIGN256((size_t)M * (size_t)K) +
                                           W8A8_ALIGN256((size_t)M * sizeof(float)));
  if (int s = hip_status(w8a8::launch_quant_rows(x, M, K, ldx, xq, a_scale, st, f16))) return s;
  return hip_status(w8a8::launch_gemm(g, st));
}

int w8a16_common(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                 const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out, int64_t ldo,
                 void* stream, bool f16) {
  if (int s = check_gemm(M, K, N, wq, w_scale, bias, out, ldo, nullptr)) return s;
  if (int s = check_bf16_ld(ldx, K)) return s;
  if (M > W8A16_MAX_M || w8a8::w8a16_lds_bytes(M, K) > w8a8::kW8A16MaxLds)
    return W8A8_ERR_UNSUPPORTED;
  if (M == 0) return W8A8_OK;
  if (!x) return W8A8_ERR_INVALID_ARG;
  if (!aligned(x, 16)) return W8A8_ERR_MISALIGNED;
  w8a8::GemmArgs g{nullptr, nullptr, wq, w_scale, bias, out, nullptr, M, N, K, ldo, f16};
  return hip_status(w8a8::launch_w8a16(x, ldx, g, (hipStream_t)stream));
}

int producer_common(const w8a8::ProducerArgs& p, void* stream) {
  if (p.M < 0) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(p.K)) return s;
  if (p.K > w8a8::kProducerMaxK[p.op]) return W8A8_ERR_UNSUPPORTED;
  if (int s = check_bf16_ld(p.ldx, p.K)) return s;
  if (p.y) {
    if (int s = check_bf16_ld(p.ldy, p.K)) return s;
  }
  const bool ln = p.op == w8a8::kProducerLayerNorm;
  if (ln) {
    if (p.rows_per_group < 1 || !(p.eps > 0.0f) || !(p.eps <= 3.4028235e38f))
      return W8A8_ERR_INVALID_ARG;
    if (int s = check_bf16_ld(p.ld_mod, p.K)) return s;
  }
  if (p.M == 0) return W8A8_OK;
  if (!p.x || !p.xq || !p.a_scale) return W8A8_ERR_INVALID_ARG;
  if (ln && (!p.shift || !p.scale)) return W8A8_ERR_INVALID_ARG;
  if (!aligned(p.x, 16) || !aligned(p.xq, 16) || !aligned(p.a_scale, 4))
    return W8A8_ERR_MISALIGNED;
  if (ln && (!aligned(p.shift, 16) || !aligned(p.scale, 16))) return W8A8_ERR_MISALIGNED;
  if (p.y && !aligned(p.y, 16)) return W8A8_ERR_MISALIGNED;
  return hip_status(w8a8::launch_producer_quant(p, (hipStream_t)stream));
}

}  // namespace

// Scratch of w8a8_linear_noalloc (the workspace w8a8_linear takes from its
// caller: xq, a_scale and any split-K partial sums). A file-scope device
// array: each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not a device
// address; its address on a device comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[W8A8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};   // address of `scratch` on each device

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with the device current) and kept.
int scratch_address(void** ptr) {
  int dev = 0;
  if (int s = hip_status(hipGetDevice(&dev))) return s;
  if (dev < 0 || dev >= kMaxDevices) return W8A8_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int s = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))) return s;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return W8A8_OK;
}

}  // namespace

extern "C" {

int w8a8_quantize_weights(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int8_t* wq,
                          float* w_scale, void* stream) {
  return quant_common(w, N, K, ldw, wq, w_scale, stream, false);
}

int w8a8_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* xq,
                   float* a_scale, void* stream) {
  return quant_common(x, M, K, ldx, xq, a_scale, stream, false);
}

int w8a8_scaled_mm(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                   const int8_t* wq, const float* w_scale, int64_t N, const uint16_t* bias,
                   uint16_t* out, int64_t ldo, int32_t* acc_debug, void* stream) {
  return scaled_mm_common(xq, a_scale, M, K, wq, w_scale, N, bias, out, ldo, acc_debug, stream,
                          false);
}

int w8a8_quantize_weights_f16(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int8_t* wq,
                              float* w_scale, void* stream) {
  return quant_common(w, N, K, ldw, wq, w_scale, stream, true);
}

int w8a8_quant_act_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* xq,
                       float* a_scale, void* stream) {
  return quant_common(x, M, K, ldx, xq, a_scale, stream, true);
}

int w8a8_scaled_mm_f16(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                       const int8_t* wq, const float* w_scale, int64_t N, const uint16_t* bias,
                       uint16_t* out, int64_t ldo, int32_t* acc_debug, void* stream) {
  return scaled_mm_common(xq, a_scale, M, K, wq, w_scale, N, bias, out, ldo, acc_debug, stream,
                          true);
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0) return 0;
  // the small-M path never splits K
  const size_t partial = (N > 0 && !small_m_path(M, K)) ? w8a8::gemm_partial_bytes(M, N, K) : 0;
  return W8A8_ALIGN256((size_t)M * (size_t)K) + W8A8_ALIGN256((size_t)M * sizeof(float)) +
         W8A8_ALIGN256(partial);
}

int w8a8_linear_path(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 1) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(K)) return s;
  if (M == 0) return W8A8_PATH_NONE;
  return small_m_path(M, K) ? W8A8_PATH_SMALL_M : W8A8_PATH_GEMM;
}

int w8a8_gemm_tile(int64_t M, int64_t K, int64_t N, int* bm, int* bn) {
  if (M < 1 || N < 1 || !bm || !bn) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(K)) return s;
  w8a8::gemm_pick_tile(M, N, K, bm, bn);
  return W8A8_OK;
}

int w8a8_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out,
                int64_t ldo, void* workspace, size_t workspace_bytes, int32_t* acc_debug,
                void* stream) {
  return linear_common(x, M, K, ldx, wq, w_scale, N, bias, out, ldo, workspace, workspace_bytes,
                       acc_debug, stream, false);
}

int w8a8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                        const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out,
                        int64_t ldo, int32_t* acc_debug, void* stream) {
  // every argument check comes before the first HIP call
  if (int s = check_gemm(M, K, N, wq, w_scale, bias, out, ldo, acc_debug)) return s;
  if (int s = check_bf16_ld(ldx, K)) return s;
  if (M == 0) return W8A8_OK;
  if (!x) return W8A8_ERR_INVALID_ARG;
  if (!aligned(x, 16)) return W8A8_ERR_MISALIGNED;
  if (w8a8_linear_workspace_bytes(M, K, N) > W8A8_NOALLOC_SCRATCH_BYTES) return W8A8_ERR_WORKSPACE;
  void* ws = nullptr;
  if (int s = scratch_address(&ws)) return s;
  return linear_common(x, M, K, ldx, wq, w_scale, N, bias, out, ldo, ws,
                       W8A8_NOALLOC_SCRATCH_BYTES, acc_debug, stream, false);
}

int w8a8_linear_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                    const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out,
                    int64_t ldo, void* workspace, size_t workspace_bytes, int32_t* acc_debug,
                    void* stream) {
  return linear_common(x, M, K, ldx, wq, w_scale, N, bias, out, ldo, workspace, workspace_bytes,
                       acc_debug, stream, true);
}

int w8a8_unpack_pack_quantized(const int32_t* packed, int64_t N, int64_t K, int64_t ldp,
                               const void* scale_in, int scale_dtype, int8_t* wq, float* w_scale,
                               void* stream) {
  if (N < 0) return W8A8_ERR_INVALID_ARG;
  if (int s = check_k(K)) return s;
  if (K > W8A8_K_MAX_PACKED) return W8A8_ERR_UNSUPPORTED;   // q = -128 needs the tighter bound
  if (ldp < K / 4) return W8A8_ERR_INVALID_ARG;
  if (ldp % 4 != 0) return W8A8_ERR_UNSUPPORTED;
  if (scale_dtype != W8A8_SCALE_F32 && scale_dtype != W8A8_SCALE_BF16 &&
      scale_dtype != W8A8_SCALE_F16)
    return W8A8_ERR_INVALID_ARG;
  if (N == 0) return W8A8_OK;
  if (!packed || !scale_in || !wq || !w_scale) return W8A8_ERR_INVALID_ARG;
  const uintptr_t salign = scale_dtype == W8A8_SCALE_F32 ? 4 : 2;
  if (!aligned(packed, 16) || !aligned(wq, 16) || !aligned(w_scale, 4) || !aligned(scale_in, salign))
    return W8A8_ERR_MISALIGNED;
  return hip_status(w8a8::launch_unpack(packed, N, K, ldp, scale_in, scale_dtype, wq, w_scale,
                                        (hipStream_t)stream));
}

int w8a16_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                 const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out, int64_t ldo,
                 void* stream) {
  return w8a16_common(x, M, K, ldx, wq, w_scale, N, bias, out, ldo, stream, false);
}

int w8a16_linear_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wq,
                     const float* w_scale, int64_t N, const uint16_t* bias, uint16_t* out,
                     int64_t ldo, void* stream) {
  return w8a16_common(x, M, K, ldx, wq, w_scale, N, bias, out, ldo, stream, true);
}

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_INVALID_ARG: return "invalid argument";
    case W8A8_ERR_UNSUPPORTED: return "unsupported shape or leading dimension";
    case W8A8_ERR_MISALIGNED: return "misaligned pointer";
    case W8A8_ERR_WORKSPACE: return "workspace missing or too small";
    case W8A8_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int w8a8_layernorm_modulate_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      const uint16_t* shift, const uint16_t* scale,
                                      int64_t ld_mod, int64_t rows_per_group, float eps,
                                      int8_t* xq, float* a_scale, uint16_t* y, int64_t ldy,
                                      void* stream) {
  w8a8::ProducerArgs p{w8a8::kProducerLayerNorm, x, M, K, ldx, shift, scale, ld_mod,
                       rows_per_group, eps, xq, a_scale, y, ldy};
  return producer_common(p, stream);
}

int w8a8_gelu_quant_act(const uint16_t* z, int64_t M, int64_t K, int64_t ldz, int approximate,
                        int8_t* xq, float* a_scale, uint16_t* y, int64_t ldy, void* stream) {
  if (approximate != W8A8_GELU_ERF && approximate != W8A8_GELU_TANH) return W8A8_ERR_INVALID_ARG;
  const int op = approximate == W8A8_GELU_ERF ? w8a8::kProducerGelu : w8a8::kProducerGeluTanh;
  w8a8::ProducerArgs p{op, z, M, K, ldz, nullptr, nullptr, 0, 1, 0.0f, xq, a_scale, y, ldy};
  return producer_common(p, stream);
}

int w8a8_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
