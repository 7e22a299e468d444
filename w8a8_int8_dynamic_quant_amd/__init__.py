"""W8A8 int8-dynamic linear layer on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libw8a8.so (C ABI in include/w8a8.h). The binding
only checks tensors and marshals device pointers and the current HIP stream;
every step of the layer runs in the library's HIP kernels. PyTorch supplies
device memory and streams. If the library is missing the functions raise:
there is no fallback.

    wq, w_scale = quantize_weights(w)              # load time, bf16/fp16 [N, K]
    y = linear(x, wq, w_scale, bias)               # bf16 [M, K] -> bf16 [M, N]
    y = linear_noalloc(x, wq, w_scale, bias, out=y)  # the same, no allocation
                                                   # (fp16 in -> fp16 out)
    xq, a_scale = quant_act(x)                     # the two ops separately
    y = scaled_mm(xq, a_scale, wq, w_scale, bias)
    wq, w_scale = unpack_pack_quantized(packed, scale)  # compressed-tensors ingest
    y = w8a16_linear(x, wq, w_scale, bias)         # weight-only, M <= 16
    xq, a_scale = layernorm_modulate_quant_act(x, shift, scale)  # fused producers
    xq, a_scale = gelu_quant_act(z)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a8.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
K_MAX = 133144
K_MAX_PACKED = 132104   # ingest: weights may hold -128
NOALLOC_SCRATCH_BYTES = 64 << 20
SMALL_M = 16          # small-M path for K <= 8192
SMALL_M_WIDE = 32     # ... and up to this M for K <= 4096
LDO_MAX = 1 << 22
PATH_NONE, PATH_SMALL_M, PATH_GEMM = 0, 1, 2
SCALE_F32, SCALE_BF16, SCALE_F16 = 0, 1, 2
W8A16_MAX_M = 16
GELU_ERF, GELU_TANH = 0, 1
PRODUCER_MAX_K = {"layernorm": 16384, "gelu": 32768}

SYMBOLS = (
    "w8a8_quantize_weights",
    "w8a8_quant_act",
    "w8a8_scaled_mm",
    "w8a8_linear",
    "w8a8_linear_noalloc",
    "w8a8_quantize_weights_f16",
    "w8a8_quant_act_f16",
    "w8a8_scaled_mm_f16",
    "w8a8_linear_f16",
    "w8a8_linear_workspace_bytes",
    "w8a8_linear_path",
    "w8a8_gemm_tile",
    "w8a8_unpack_pack_quantized",
    "w8a16_linear",
    "w8a16_linear_f16",
    "w8a8_layernorm_modulate_quant_act",
    "w8a8_gelu_quant_act",
    "w8a8_status_string",
    "w8a8_last_hip_error",
)

_lib = None


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        msg = f"{fn}: {status_string(status)} (status {status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """The loaded libw8a8.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m w8a8_int8_dynamic_quant_amd.build_lib` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    ci = ctypes.c_int
    L.w8a8_quantize_weights.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    L.w8a8_quant_act.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    L.w8a8_scaled_mm.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, i64, vp, vp]
    L.w8a8_linear.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp, i64, vp, sz, vp, vp]
    L.w8a8_linear_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp, i64, vp, vp]
    L.w8a8_quantize_weights_f16.argtypes = L.w8a8_quantize_weights.argtypes
    L.w8a8_quant_act_f16.argtypes = L.w8a8_quant_act.argtypes
    L.w8a8_scaled_mm_f16.argtypes = L.w8a8_scaled_mm.argtypes
    L.w8a8_linear_f16.argtypes = L.w8a8_linear.argtypes
    L.w8a8_linear_workspace_bytes.argtypes = [i64, i64, i64]
    L.w8a8_linear_workspace_bytes.restype = sz
    L.w8a8_linear_path.argtypes = [i64, i64, i64]
    L.w8a8_gemm_tile.argtypes = [i64, i64, i64, ctypes.POINTER(ci), ctypes.POINTER(ci)]
    L.w8a8_unpack_pack_quantized.argtypes = [vp, i64, i64, i64, vp, ci, vp, vp, vp]
    L.w8a16_linear.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp, i64, vp]
    L.w8a16_linear_f16.argtypes = L.w8a16_linear.argtypes
    L.w8a8_layernorm_modulate_quant_act.argtypes = [vp, i64, i64, i64, vp, vp, i64, i64,
                                                    ctypes.c_float, vp, vp, vp, i64, vp]
    L.w8a8_gelu_quant_act.argtypes = [vp, i64, i64, i64, ci, vp, vp, vp, i64, vp]
    L.w8a8_status_string.argtypes = [ci]
    L.w8a8_status_string.restype = ctypes.c_char_p
    L.w8a8_last_hip_error.argtypes = []
    for name in ("w8a8_quantize_weights", "w8a8_quant_act", "w8a8_scaled_mm", "w8a8_linear",
                 "w8a8_linear_noalloc",
                 "w8a8_quantize_weights_f16", "w8a8_quant_act_f16", "w8a8_scaled_mm_f16",
                 "w8a8_linear_f16",
                 "w8a8_linear_path", "w8a8_gemm_tile", "w8a8_unpack_pack_quantized", "w8a16_linear",
                 "w8a16_linear_f16", "w8a8_layernorm_modulate_quant_act", "w8a8_gelu_quant_act",
                 "w8a8_last_hip_error"):
        getattr(L, name).restype = ci
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().w8a8_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        detail = ""
        if status == ERR_HIP:
            detail = f"hipError {lib().w8a8_last_hip_error()}"
        raise W8A8Error(fn, status, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _rows(t: torch.Tensor, dtype, name: str):
    """(rows, cols, leading dim) of a 2-D tensor with unit column stride."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.shape[0] > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return t.shape[0], t.shape[1], ld


# 16-bit floating-point types of x / w / bias / out and the entry-point suffix
_HALF = {torch.bfloat16: "", torch.float16: "_f16"}


def _half(dtype, name: str) -> str:
    if dtype not in _HALF:
        raise TypeError(f"{name} must be bfloat16 or float16, got {dtype}")
    return _HALF[dtype]


def _vec(t, dtype, n, name):
    if t is None:
        return None
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] != n or not t.is_cuda:
        raise ValueError(f"{name} must be a {dtype} GPU vector of length {n}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def quantize_weights(w: torch.Tensor):
    """bf16 or fp16 W [N, K] -> (wq int8 [N, K], w_scale fp32 [N])."""
    fn = "w8a8_quantize_weights" + _half(w.dtype, "w")
    N, K, ld = _rows(w, w.dtype, "w")
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    s = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check(fn, getattr(lib(), fn)(_ptr(w), N, K, ld, _ptr(wq), _ptr(s), _stream(w.device)))
    return wq, s


def quant_act(x: torch.Tensor):
    """bf16 or fp16 x [M, K] -> (xq int8 [M, K], a_scale fp32 [M])."""
    fn = "w8a8_quant_act" + _half(x.dtype, "x")
    M, K, ld = _rows(x, x.dtype, "x")
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(fn, getattr(lib(), fn)(_ptr(x), M, K, ld, _ptr(xq), _ptr(s), _stream(x.device)))
    return xq, s


def scaled_mm(xq, a_scale, wq, w_scale, bias=None, out=None, acc_debug=None,
              dtype=torch.bfloat16):
    """int8 xq [M,K] x int8 wq [N,K] -> [M,N] of `dtype` (bf16 or fp16; the
    type of `out` when given) with the scale epilogue; bias has that type.

    acc_debug: optional int32 [M, N] tensor that receives the raw
    accumulators from the same kernel.
    """
    if out is not None:
        dtype = out.dtype
    fn = "w8a8_scaled_mm" + _half(dtype, "out")
    M, K, ldq = _rows(xq, torch.int8, "xq")
    N, K2, ldw = _rows(wq, torch.int8, "wq")
    if K2 != K or (M > 1 and ldq != K) or (N > 1 and ldw != K):
        raise ValueError("xq and wq must be contiguous [*, K] with the same K")
    _vec(a_scale, torch.float32, M, "a_scale")
    _vec(w_scale, torch.float32, N, "w_scale")
    _vec(bias, dtype, N, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=xq.device)
    Mo, No, ldo = _rows(out, dtype, "out")
    if (Mo, No) != (M, N):
        raise ValueError("out must be [M, N]")
    if acc_debug is not None and (acc_debug.shape != (M, N) or acc_debug.dtype != torch.int32
                                  or not acc_debug.is_contiguous()):
        raise ValueError("acc_debug must be a contiguous int32 [M, N] tensor")
    _check(fn, getattr(lib(), fn)(_ptr(xq), _ptr(a_scale), M, K, _ptr(wq), _ptr(w_scale), N,
                                  _ptr(bias), _ptr(out), ldo, _ptr(acc_debug),
                                  _stream(xq.device)))
    return out


_SCALE_DTYPES = {torch.float32: SCALE_F32, torch.bfloat16: SCALE_BF16, torch.float16: SCALE_F16}


def unpack_pack_quantized(packed: torch.Tensor, scale: torch.Tensor):
    """compressed-tensors pack-quantized weights -> (wq int8 [N, K], w_scale fp32 [N]).

    packed: int32 [N, K/4] (bytes offset by 128, four to a word, little-endian);
    scale: fp32, bf16 or fp16 of N elements ([N] or [N, 1]).
    """
    N, words, ldp = _rows(packed, torch.int32, "packed")
    K = 4 * words
    if scale.dtype not in _SCALE_DTYPES or scale.numel() != N or not scale.is_cuda:
        raise ValueError("scale must be a fp32/bf16/fp16 GPU tensor of N elements")
    scale = scale.reshape(N)
    if not scale.is_contiguous():
        raise ValueError("scale must be contiguous")
    wq = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    s = torch.empty((N,), dtype=torch.float32, device=packed.device)
    _check("w8a8_unpack_pack_quantized",
           lib().w8a8_unpack_pack_quantized(_ptr(packed), N, K, ldp, _ptr(scale),
                                            _SCALE_DTYPES[scale.dtype], _ptr(wq), _ptr(s),
                                            _stream(packed.device)))
    return wq, s


def w8a16_linear(x, wq, w_scale, bias=None, out=None):
    """W8A16 linear for M <= 16: bf16 (or fp16) x [M, K] (not quantised) with
    int8 weights [N, K] and fp32 per-channel scales -> [M, N] of x's type."""
    fn = "w8a16_linear" + _half(x.dtype, "x")
    M, K, ldx = _rows(x, x.dtype, "x")
    N, K2, ldw = _rows(wq, torch.int8, "wq")
    if K2 != K or (N > 1 and ldw != K):
        raise ValueError("wq must be contiguous [N, K] with the K of x")
    _vec(w_scale, torch.float32, N, "w_scale")
    _vec(bias, x.dtype, N, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    Mo, No, ldo = _rows(out, x.dtype, "out")
    if (Mo, No) != (M, N):
        raise ValueError("out must be [M, N]")
    _check(fn, getattr(lib(), fn)(_ptr(x), M, K, ldx, _ptr(wq), _ptr(w_scale), N, _ptr(bias),
                                  _ptr(out), ldo, _stream(x.device)))
    return out


def workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().w8a8_linear_workspace_bytes(M, K, N))


def linear_path(M: int, K: int, N: int) -> int:
    return int(lib().w8a8_linear_path(M, K, N))


def gemm_tile(M: int, K: int, N: int):
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    _check("w8a8_gemm_tile", lib().w8a8_gemm_tile(M, K, N, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def workspace_views(workspace: torch.Tensor, M: int, K: int):
    """(xq [M,K] int8, a_scale [M] fp32) views of a linear() workspace."""
    off = (M * K + 255) // 256 * 256
    xq = workspace[: M * K].view(torch.int8).view(M, K)
    sa = workspace[off: off + 4 * M].view(torch.float32)
    return xq, sa


def linear(x, wq, w_scale, bias=None, out=None, workspace=None, acc_debug=None):
    """W8A8 linear: bf16 x [M, K] -> bf16 [M, N] (fp16 x -> fp16 y; bias and
    out have the type of x).

    workspace: optional uint8 GPU tensor of at least workspace_bytes(M,K,N)
    bytes; after the call it holds xq and a_scale (see workspace_views).
    """
    fn = "w8a8_linear" + _half(x.dtype, "x")
    M, K, ldx = _rows(x, x.dtype, "x")
    N, K2, ldw = _rows(wq, torch.int8, "wq")
    if K2 != K or (N > 1 and ldw != K):
        raise ValueError("wq must be contiguous [N, K] with the K of x")
    _vec(w_scale, torch.float32, N, "w_scale")
    _vec(bias, x.dtype, N, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    Mo, No, ldo = _rows(out, x.dtype, "out")
    if (Mo, No) != (M, N):
        raise ValueError("out must be [M, N]")
    need = workspace_bytes(M, K, N)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if acc_debug is not None and (acc_debug.shape != (M, N) or acc_debug.dtype != torch.int32
                                  or not acc_debug.is_contiguous()):
        raise ValueError("acc_debug must be a contiguous int32 [M, N] tensor")
    _check(fn, getattr(lib(), fn)(_ptr(x), M, K, ldx, _ptr(wq), _ptr(w_scale), N, _ptr(bias),
                                  _ptr(out), ldo, _ptr(workspace), workspace.numel(),
                                  _ptr(acc_debug), _stream(x.device)))
    return out


def linear_noalloc(x, wq, w_scale, bias=None, out=None, acc_debug=None):
    """W8A8 linear (bf16 x [M, K] -> bf16 [M, N]) through
    w8a8_linear_noalloc: the library's per-GPU scratch array replaces the
    workspace, so the call allocates nothing when `out` is given (for callers
    that cannot allocate). Calls that overlap on one GPU share that scratch
    and must be serialised by the caller."""
    if x.dtype != torch.bfloat16:
        raise TypeError("linear_noalloc takes bf16 activations")
    M, K, ldx = _rows(x, x.dtype, "x")
    N, K2, ldw = _rows(wq, torch.int8, "wq")
    if K2 != K or (N > 1 and ldw != K):
        raise ValueError("wq must be contiguous [N, K] with the K of x")
    _vec(w_scale, torch.float32, N, "w_scale")
    _vec(bias, x.dtype, N, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    Mo, No, ldo = _rows(out, x.dtype, "out")
    if (Mo, No) != (M, N):
        raise ValueError("out must be [M, N]")
    if acc_debug is not None and (acc_debug.shape != (M, N) or acc_debug.dtype != torch.int32
                                  or not acc_debug.is_contiguous()):
        raise ValueError("acc_debug must be a contiguous int32 [M, N] tensor")
    _check("w8a8_linear_noalloc",
           lib().w8a8_linear_noalloc(_ptr(x), M, K, ldx, _ptr(wq), _ptr(w_scale), N, _ptr(bias),
                                     _ptr(out), ldo, _ptr(acc_debug), _stream(x.device)))
    return out


def _producer_out(x, M, K, return_y):
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty((M,), dtype=torch.float32, device=x.device)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if return_y else None
    return xq, s, y


def layernorm_modulate_quant_act(x, shift, scale, eps: float = 1e-6, rows_per_group=None,
                                 return_y: bool = False):
    """Modulated LayerNorm of bf16 x [M, K] fused with its per-row int8
    quantisation: (x - mean) / sqrt(var + eps) * (1 + scale) + shift, rounded
    to bf16, then quantised -> (xq int8 [M, K], a_scale fp32 [M][, y bf16]).

    shift, scale: bf16 [K] (every row) or [G, K] with the same row stride
    (e.g. chunks of a modulation projection's output); row m uses group
    m // rows_per_group (default: M / G, which must then divide evenly).
    """
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    if shift.dim() == 1:
        shift, scale = shift.unsqueeze(0), scale.unsqueeze(0)
    G, Ks, ldm = _rows(shift, torch.bfloat16, "shift")
    G2, Kc, ldm2 = _rows(scale, torch.bfloat16, "scale")
    if (G2, Kc) != (G, Ks) or Ks != K:
        raise ValueError("shift and scale must both be [K] or [G, K] with the K of x")
    if G > 1 and ldm2 != ldm:
        raise ValueError("shift and scale must have the same row stride")
    if rows_per_group is None:
        if M % G:
            raise ValueError("pass rows_per_group when G does not divide M")
        rows_per_group = max(M // G, 1)
    if M and -(-M // rows_per_group) > G:
        raise ValueError(f"{-(-M // rows_per_group)} row groups need that many shift/scale rows")
    xq, s, y = _producer_out(x, M, K, return_y)
    _check("w8a8_layernorm_modulate_quant_act",
           lib().w8a8_layernorm_modulate_quant_act(
               _ptr(x), M, K, ldx, _ptr(shift), _ptr(scale), ldm if G > 1 else K,
               int(rows_per_group), float(eps), _ptr(xq), _ptr(s), _ptr(y), K,
               _stream(x.device)))
    return (xq, s, y) if return_y else (xq, s)


def gelu_quant_act(z, approximate: str = "none", return_y: bool = False):
    """GELU of bf16 z [M, K] ('none': z Phi(z); 'tanh': the tanh form) fused
    with its per-row int8 quantisation -> (xq, a_scale[, y bf16])."""
    codes = {"none": GELU_ERF, "tanh": GELU_TANH}
    if approximate not in codes:
        raise ValueError("approximate must be 'none' or 'tanh'")
    M, K, ldz = _rows(z, torch.bfloat16, "z")
    xq, s, y = _producer_out(z, M, K, return_y)
    _check("w8a8_gelu_quant_act",
           lib().w8a8_gelu_quant_act(_ptr(z), M, K, ldz, codes[approximate], _ptr(xq), _ptr(s),
                                     _ptr(y), K, _stream(z.device)))
    return (xq, s, y) if return_y else (xq, s)
