/*
 * w8a8.h - C ABI of libw8a8, the W8A8 int8-dynamic linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (sources are the pages' titles and sections):
 *
 *   y[m,n] = bf16( ((fl32(acc[m,n]) * a_scale[m]) * w_scale[n]) + bias[n] )
 *   acc[m,n] = sum_k xq[m,k] * wq[n,k]                 (exact, int32)
 *   xq, a_scale = per-row symmetric int8 quantisation of x (dynamic)
 *   wq, w_scale = per-row symmetric int8 quantisation of W (load time)
 *
 * - "Issue 5 probe: int8 quantized DiT serve paths on the RTX 3090 (24 GB)",
 *   section "Round two ... W8A8 int8-dynamic": int8 weights, dynamic
 *   per-token symmetric int8 activations, an int8 scaled matrix product; the
 *   stored artifact is unpacked int8 weights plus fp32 per-channel scales;
 *   the result carries act_scale.
 * - "Int8 Quantization" (vLLM-Omni user guide), "Overview" and "Parameters":
 *   weights are quantised at load time or loaded pre-quantised; activation
 *   scaling is dynamic only.
 * - unsloth test_diffusion_transformer_quant.py commit log: int8 products
 *   accumulate in int32; the torch._int_mm route needs M > 16 and so could
 *   not serve the M = 1 modulation projections. This library has no such
 *   limit: M <= W8A8_SMALL_M (M <= W8A8_SMALL_M_WIDE for K <= 4096) goes to
 *   a bandwidth-bound small-M kernel.
 *
 * Per-row quantisation of a row r[0..K-1]:
 *   amax = max_k |r[k]|,  scale = fl32(amax / 127)   (IEEE fp32 division)
 *   q[k] = clamp(round_half_even(fl32(r[k] / scale)), -127, 127)
 *   an all-zero row gives scale = 0 and q = 0.
 *
 * Conventions for every entry point:
 * - Pointers are DEVICE pointers owned by the caller. The library allocates
 *   nothing, keeps no state between calls, is reentrant, never writes its
 *   inputs, and only enqueues work on `stream` (a hipStream_t passed as
 *   void*; NULL = the default stream). A call returns once the work is
 *   enqueued; the caller keeps every buffer alive until the stream has run it.
 * - One file-scope device array is the exception to "no state": the 64 MiB
 *   scratch of w8a8_linear_noalloc (see there), which each GPU the library
 *   runs on holds until the process ends. (The 256 KiB GELU lookup table of
 *   w8a8_gelu_quant_act is read-only data built into the library.)
 * - Layouts are row-major. bf16 values are passed as uint16_t bit patterns.
 * - Arguments are validated before anything is launched; on an error nothing
 *   is enqueued and an error status is returned (no exceptions, no abort).
 * - Requirements: M >= 0 (M == 0 is a no-op), N >= 1, 16 <= K <= W8A8_K_MAX
 *   and K % 16 == 0 (else W8A8_ERR_UNSUPPORTED); every leading dimension
 *   ld >= K (ldo >= N, ldo <= W8A8_LDO_MAX); bf16 input leading dimensions
 *   are multiples of 8;
 *   x/w/xq/wq/workspace pointers 16-byte aligned, scale/bias/out/acc_debug
 *   pointers 4-byte aligned (else W8A8_ERR_MISALIGNED).
 * - Outputs are undefined if an output buffer overlaps any other buffer.
 * - Subnormal inputs are legal and never flushed. NaN/Inf inputs are
 *   outside the contract: no fault, unspecified values.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_INVALID_ARG = -1,  /* NULL pointer, negative size, ld too small  */
  W8A8_ERR_UNSUPPORTED = -2,  /* K % 16 != 0, K > W8A8_K_MAX, odd ld        */
  W8A8_ERR_MISALIGNED = -3,   /* pointer alignment below the requirement    */
  W8A8_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than required    */
  W8A8_ERR_HIP = -5           /* a HIP launch failed; see w8a8_last_hip_error */
} w8a8_status;

/* Largest K whose worst-case accumulator 127*127*K fits in int32. */
#define W8A8_K_MAX 133144
/* Rows up to this count take the small-M (weight-streaming) path when
 * K <= 8192; up to W8A8_SMALL_M_WIDE rows take it when K <= 4096. */
#define W8A8_SMALL_M 16
#define W8A8_SMALL_M_WIDE 32
/* Largest output leading dimension (elements; the debug accumulators allow
 * N up to half of it): kernels address a 256-row output tile with 32-bit
 * byte offsets. Larger values give W8A8_ERR_UNSUPPORTED. */
#define W8A8_LDO_MAX (1 << 22)

/*
 * Load-time per-output-channel weight quantisation ("Int8 Quantization"
 * guide, "Overview": bf16 and fp16 weights quantised at load time; Issue 5 probe,
 * "Round two": unpacked int8 weights plus fp32 per-channel scales).
 *   w        [N, ldw] bf16 (read)
 *   wq       [N, K] int8, row stride K (written)
 *   w_scale  [N] fp32 (written)
 * The weight layout stays [N, K] with K contiguous: no transpose or repack
 * is needed afterwards, both GEMM operands are K-contiguous.
 */
int w8a8_quantize_weights(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                          int8_t* wq, float* w_scale, void* stream);

/*
 * Dynamic per-token activation quantisation (Issue 5 probe, "Round two":
 * dynamic per-token symmetric int8 activations).
 *   x        [M, ldx] bf16 (read)
 *   xq       [M, K] int8, row stride K (written)
 *   a_scale  [M] fp32 (written)
 */
int w8a8_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                   int8_t* xq, float* a_scale, void* stream);

/*
 * Scaled int8 matrix product on pre-quantised activations (the second of the
 * two ops of Issue 5 probe, "Round two": the int8 scaled-MM).
 *   xq [M, K] int8 (row stride K), a_scale [M] fp32
 *   wq [N, K] int8 (row stride K), w_scale [N] fp32
 *   bias [N] bf16 or NULL
 *   out [M, ldo] bf16 (written)
 *   acc_debug [M, N] int32 (row stride N) or NULL: when given, the same
 *     kernel also stores its raw int32 accumulators there (for parity checks).
 */
int w8a8_scaled_mm(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                   const int8_t* wq, const float* w_scale, int64_t N,
                   const uint16_t* bias, uint16_t* out, int64_t ldo,
                   int32_t* acc_debug, void* stream);

/*
 * The whole W8A8 linear: dynamic activation quantisation, int8 product and
 * scale epilogue.
 *   x [M, ldx] bf16; wq [N, K] int8; w_scale [N] fp32; bias [N] bf16 or NULL
 *   out [M, ldo] bf16 (written)
 *   workspace: device scratch of at least w8a8_linear_workspace_bytes(M,K,N)
 *     bytes, 16-byte aligned, owned by the caller. After the call it holds the
 *     quantised activations xq [M, K] int8 (row stride K) at byte offset 0 and
 *     a_scale [M] fp32 at byte offset W8A8_ALIGN256(M*K), on both paths.
 *     For shapes whose 128x128 tiles fill at most one round of the compute
 *     units (N % 8 == 0, K above 896; w8a8_gemm_tile reports the tile), and
 *     for 64x64 tiles numbering up to two per compute unit (K of at least
 *     1024), when the shape is not on the small-M path, the size also covers
 *     two to four slices of int32 partial sums after a_scale: the GEMM then
 *     splits K and a second kernel adds the partial sums before the
 *     epilogue (exact in int32, so the results are the same bits). The size
 *     depends on the current device's compute-unit count.
 *   acc_debug [M, N] int32 or NULL, as in w8a8_scaled_mm.
 * Path: M <= W8A8_SMALL_M with K <= 8192, or M <= W8A8_SMALL_M_WIDE with
 * K <= 4096, runs one fused weight-streaming kernel that quantises x on chip; otherwise the activation quantisation
 * kernel runs first and the MFMA GEMM second (split as above where the
 * workspace holds the partial sums and the output rows are 16-byte aligned
 * with ldo % 8 == 0). All paths give bit-identical xq, a_scale, acc and out
 * for the same row.
 */
int w8a8_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                const int8_t* wq, const float* w_scale, int64_t N,
                const uint16_t* bias, uint16_t* out, int64_t ldo,
                void* workspace, size_t workspace_bytes,
                int32_t* acc_debug, void* stream);

#define W8A8_ALIGN256(b) ((((size_t)(b)) + 255u) & ~(size_t)255u)

/*
 * w8a8_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer, the same kernels and bits, with the workspace taken from a
 * file-scope device array of W8A8_NOALLOC_SCRATCH_BYTES (64 MiB) instead of
 * the caller. The caller still passes x, the weights, out and acc_debug.
 * - Each GPU the library runs on holds its own copy of the array until the
 *   process ends; the first call on a device looks up the array's address on
 *   that device (hipGetSymbolAddress) and keeps it.
 * - No call allocates or frees memory (no hipMalloc, no hipFree, no
 *   allocating library routine).
 * - Every call on one GPU shares that GPU's array and leaves its contents
 *   behind (xq at byte offset 0, a_scale at W8A8_ALIGN256(M*K)): calls whose
 *   work overlaps on one GPU (different streams, or host threads) race on it
 *   and must be serialised by the caller. Nothing in it needs clearing: every
 *   byte a call reads, the same call writes first.
 * - Shapes whose w8a8_linear_workspace_bytes(M, K, N) exceeds the array are
 *   refused with W8A8_ERR_WORKSPACE (every 1024 px DiT block linear fits);
 *   other requirements and errors as w8a8_linear.
 */
#define W8A8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w8a8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        const int8_t* wq, const float* w_scale, int64_t N,
                        const uint16_t* bias, uint16_t* out, int64_t ldo,
                        int32_t* acc_debug, void* stream);

/*
 * fp16 variants ("Int8 Quantization" guide, "Overview": bf16 and fp16 weights
 * are quantised at load time; Issue 5 probe, "Round one": the layers run with
 * bf16 and with fp16 activations). Each has the signature, layouts,
 * requirements and errors of the bf16 entry point of the same name, with
 * every 16-bit floating-point buffer (w, x, bias, out) holding IEEE binary16
 * bit patterns instead of bf16. The arithmetic is the same: inputs convert
 * exactly to fp32; scales are fp32; y = fp16_round_to_nearest_even(
 * ((fl32(acc) * a_scale) * w_scale) + bias), subnormal results kept, and a
 * value past the largest finite fp16 (65504; from 65520 up) becomes +-inf.
 * wq / w_scale / xq / a_scale are the same int8 / fp32 buffers as for bf16,
 * so weights prepared by either quantiser serve either type.
 */
int w8a8_quantize_weights_f16(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                              int8_t* wq, float* w_scale, void* stream);
int w8a8_quant_act_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                       int8_t* xq, float* a_scale, void* stream);
int w8a8_scaled_mm_f16(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                       const int8_t* wq, const float* w_scale, int64_t N,
                       const uint16_t* bias, uint16_t* out, int64_t ldo,
                       int32_t* acc_debug, void* stream);
int w8a8_linear_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                    const int8_t* wq, const float* w_scale, int64_t N,
                    const uint16_t* bias, uint16_t* out, int64_t ldo,
                    void* workspace, size_t workspace_bytes,
                    int32_t* acc_debug, void* stream);

/*
 * compressed-tensors pack-quantized ingest (Issue 5 probe, "Round one: int8
 * weight-only via compressed-tensors": weights stored with pack_to_int32, as
 * unsigned bytes offset by 128, four to a 32-bit word).
 *   packed   [N, ldp] int32 (read); element 4i+j of a row is bits 8j..8j+7 of
 *            word i (little-endian), stored as q + 128
 *   scale_in [N] per-output-channel scale, type scale_dtype (W8A8_SCALE_F32,
 *            W8A8_SCALE_BF16 or W8A8_SCALE_F16) (read)
 *   wq       [N, K] int8, row stride K (written): q = stored byte - 128
 *   w_scale  [N] fp32 (written; every input type converts exactly)
 * The result feeds w8a8_linear / w8a8_scaled_mm like the output of
 * w8a8_quantize_weights. Requirements: 16 <= K <= W8A8_K_MAX_PACKED, K % 16
 * == 0, ldp >= K/4 and ldp % 4 == 0 (else W8A8_ERR_UNSUPPORTED /
 * INVALID_ARG); packed and wq 16-byte aligned. A stored byte 0 gives q = -128,
 * which the symmetric quantiser never produces; with such weights the
 * int32-safe K is W8A8_K_MAX_PACKED (127 * 128 * K < 2^31) rather than
 * W8A8_K_MAX, so longer rows are refused with W8A8_ERR_UNSUPPORTED.
 */
#define W8A8_K_MAX_PACKED 132104
#define W8A8_SCALE_F32 0
#define W8A8_SCALE_BF16 1
#define W8A8_SCALE_F16 2
int w8a8_unpack_pack_quantized(const int32_t* packed, int64_t N, int64_t K, int64_t ldp,
                               const void* scale_in, int scale_dtype, int8_t* wq,
                               float* w_scale, void* stream);

/*
 * W8A16 linear for small M: int8 weight-only with bf16 activations, no
 * activation quantisation (Issue 5 probe, "Round one: int8 weight-only via
 * compressed-tensors": per-output-channel symmetric int8 weights, bf16
 * activations), for the M <= 16 layers that stream their weight once.
 *   x [M, ldx] bf16; wq [N, K] int8 (row stride K); w_scale [N] fp32
 *   (from w8a8_quantize_weights or w8a8_unpack_pack_quantized);
 *   bias [N] bf16 or NULL; out [M, ldo] bf16 (written)
 *   acc[m,n] = sum_k fp32(x[m,k]) * wq[n,k]   (fp32 accumulation, MFMA order)
 *   y[m,n]   = bf16_rne(fl32(acc * w_scale[n]) + bias[n])
 * Requirements as w8a8_linear, plus M <= W8A16_MAX_M and K small enough that
 * the activations fit on chip: K <= 8064 for M <= 8, K <= 3968 for M <= 16
 * (else W8A8_ERR_UNSUPPORTED). No workspace.
 */
#define W8A16_MAX_M 16
int w8a16_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                 const int8_t* wq, const float* w_scale, int64_t N,
                 const uint16_t* bias, uint16_t* out, int64_t ldo, void* stream);
/* The same with fp16 activations, bias and output (the probe's Round one ran
 * the weight-only layers with bf16 and with fp16 activations):
 *   y = fp16_rne(fl32(acc * w_scale[n]) + bias[n]), acc = sum_k fp32(x) * wq
 * (every fp16 x int8 product is exact in fp32); subnormal results kept,
 * overflow to +-inf. Requirements and errors as w8a16_linear. */
int w8a16_linear_f16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     const int8_t* wq, const float* w_scale, int64_t N,
                     const uint16_t* bias, uint16_t* out, int64_t ldo, void* stream);

/*
 * Producers fused with the activation quantisation ("Qwen-Image-2.1: TE
 * AutoRound-AWQ on GPU + all-resident single-3090 stack", section
 * "Whole-pipeline follow-up": the W8A8 DiT path runs fused
 * activation-quantisation, normalisation and activation kernels around its
 * int8 GEMMs). Each computes the producer's bf16 row y in registers and
 * writes the per-row quantisation of y, bit for bit what w8a8_quant_act
 * writes for y, without a bf16 round trip through memory. y itself is also
 * written when a y pointer is given (else pass NULL; ldy is then ignored).
 *   xq      [M, K] int8, row stride K (written)
 *   a_scale [M] fp32 (written)
 *   y       [M, ldy] bf16 (written) or NULL
 * y is the fp32 evaluation of the formula rounded to bf16 (nearest even):
 * within half a bf16 ulp of the exact value plus the fp32 rounding error.
 * Requirements as w8a8_quant_act (16 <= K, K % 16 == 0, ld >= K and
 * ld % 8 == 0, x / xq / y 16-byte aligned, a_scale 4-byte aligned), plus
 * the per-producer limits below; ldy follows the rules of ldx when y is
 * given. No workspace.
 */

/*
 * Modulated (adaptive) LayerNorm, the normalisation in front of a DiT
 * block's QKV and FFN-up linears:
 *   y[m,k] = bf16((x[m,k] - mean_m) / sqrt(var_m + eps) * (1 + scale[g,k]) + shift[g,k])
 * mean_m and the biased variance var_m over row m of x; g = m / rows_per_group
 * (the tokens of one sample share a group's shift and scale).
 *   x            [M, ldx] bf16 (read)
 *   shift, scale [G, ld_mod] bf16 (read), G = ceil(M / rows_per_group)
 * fp32 evaluation: every term of the two row sums passes through at most
 * K / 64 + 16 additions; mean = sum / K, rstd = 1 / sqrt(var + eps).
 * Limits: K <= 16384 (else W8A8_ERR_UNSUPPORTED); eps > 0 and finite,
 * rows_per_group >= 1, ld_mod >= K (else W8A8_ERR_INVALID_ARG); ld_mod % 8
 * == 0 (else W8A8_ERR_UNSUPPORTED); shift and scale 16-byte aligned.
 */
int w8a8_layernorm_modulate_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      const uint16_t* shift, const uint16_t* scale,
                                      int64_t ld_mod, int64_t rows_per_group, float eps,
                                      int8_t* xq, float* a_scale, uint16_t* y, int64_t ldy,
                                      void* stream);

/*
 * GELU, the activation in front of a DiT block's FFN-down linear:
 *   W8A8_GELU_ERF:  y = bf16(z Phi(z)), Phi the standard normal distribution
 *                   function;
 *   W8A8_GELU_TANH: y = bf16(0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))).
 *   y is the bf16 nearest to GELU(z) (half to even) as evaluated in double
 *   precision: the library carries the whole bf16 -> bf16 map of each form,
 *   computed at build time, and looks every element up.
 *   z [M, ldz] bf16 (read)
 * Limits: K <= 32768 (else W8A8_ERR_UNSUPPORTED); approximate one of the two
 * values (else W8A8_ERR_INVALID_ARG).
 */
#define W8A8_GELU_ERF 0
#define W8A8_GELU_TANH 1
int w8a8_gelu_quant_act(const uint16_t* z, int64_t M, int64_t K, int64_t ldz, int approximate,
                        int8_t* xq, float* a_scale, uint16_t* y, int64_t ldy, void* stream);

/* Workspace bytes w8a8_linear needs for this shape (0 if M == 0). */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* Which kernels w8a8_linear runs for this shape: W8A8_PATH_SMALL_M (fused
 * small-M kernel) or W8A8_PATH_GEMM (quantisation kernel + MFMA GEMM);
 * W8A8_PATH_NONE for M == 0; a negative w8a8_status for invalid sizes. */
#define W8A8_PATH_NONE 0
#define W8A8_PATH_SMALL_M 1
#define W8A8_PATH_GEMM 2
int w8a8_linear_path(int64_t M, int64_t K, int64_t N);

/* The GEMM tile configuration the MFMA kernel uses for this shape
 * (BM rows of x by BN rows of W per workgroup), for checking kernel choice. */
int w8a8_gemm_tile(int64_t M, int64_t K, int64_t N, int* bm, int* bn);

/* Static text for a status code. */
const char* w8a8_status_string(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int w8a8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
