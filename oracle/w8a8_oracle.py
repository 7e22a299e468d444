"""Plain, slow CPU oracle of the W8A8 int8-dynamic linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What is computed (y = W8A8 linear of bf16 activations x [M,K] and bf16
weights W [N,K]):

  1. per-token (per-row) symmetric int8 quantisation of x with
     scale = amax/127,
  2. per-output-channel symmetric int8 quantisation of W with an fp32 scale
     per output channel,
  3. an int8 x int8 product with exact integer accumulation, stored as int32,
  4. an fp32 epilogue acc * act_scale * weight_scale (+ bias) rounded to bf16.

and, for the producers fused with step 1, the modulated LayerNorm and the GELU
whose bf16 output is quantised in the same pass (the last section).

Sources (page titles and sections; the pages are the authority):

* "Issue 5 probe: int8 quantized DiT serve paths on the RTX 3090 (24 GB)",
  section "Round two ... W8A8 int8-dynamic": int8 weights with dynamic
  per-token symmetric int8 activations, served by an int8 scaled-MM; the
  artifact stores unpacked int8 weights with fp32 per-channel scales; the
  probe's reference has to carry the act_scale factor (the 97% error scare
  was that factor missing). Section "Kernel isolation": the reference the
  layer is compared against is float32 x @ dequant(W)^T.
* "Int8 Quantization" (vLLM-Omni user guide), sections "Overview" and
  "Parameters": bf16 and fp16 weights are quantised at load time; only dynamic
  (online) activation scaling exists.
* "Qwen-Image-2.1: TE AutoRound-AWQ on GPU + all-resident single-3090 stack",
  section "Whole-pipeline follow-up": per-token activation and per-channel
  weight quantisation.
* unsloth commit log of test_diffusion_transformer_quant.py: int8 matmuls run
  with int32 accumulation.
* "Qwen-Image-2.1 ...", section "Whole-pipeline follow-up": fused
  activation-quantisation, normalisation and activation kernels around the
  int8 GEMMs (the producers of the last section).

Readings where the pages are silent (each is a choice this oracle fixes and
the HIP path must reproduce):

* scale = fl32(amax / 127) by one IEEE fp32 division; q = fl32(x / scale)
  by a second IEEE fp32 division, then round half to even, then clamp to
  [-127, 127] (symmetric: -128 is never produced).
* all-zero row: scale = 0 and q = 0.
* both scales are fp32.
* epilogue order ((fl32(acc) * s_a) * s_w) + fp32(bias), each step rounded
  to fp32 (no fused multiply-add), then bf16 round to nearest even.
* bias is optional and added after both scales.
* the integer product is exact; |acc| <= 127^2 K must fit int32, so
  K <= 133 144.
* subnormal inputs are legal and are not flushed; NaN/Inf inputs are outside
  the contract.
* fp16 activations, weights, bias and output (the guide quantises bf16 and
  fp16 weights; the Issue 5 probe, "Round one", runs bf16 and fp16 activations):
  the same maths with fp16 in place of bf16. Inputs convert exactly to fp32;
  y is the fp16 round to nearest even of the same fp32 value, and a value
  past the largest finite fp16 rounds to infinity as IEEE rounding does.

Parity pins: every function here is checked by tests that do not call it
back (hand-computed golden files, exact rational arithmetic, brute force,
closed forms, invariants, a library cast, the pages' 0.17% figure, and for
the producers the standard normal table and independent library
implementations of LayerNorm, GELU and erfc). No function is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

# |acc| <= 127 * 127 * K must fit in int32.
K_MAX = (2**31 - 1) // (127 * 127)          # 133 144

_F32_127 = np.float32(127.0)


# --- bf16 <-> fp32 -------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(t) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit and dropping the low 16 bits is
    RNE on the magnitude; overflow past the largest finite value carries into
    the exponent and gives infinity, as IEEE rounding does. NaN stays NaN.
    """
    f = np.asarray(t, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)
    return r


# --- fp16 <-> fp32 -------------------------------------------------------

def f16_bits_to_f32(bits) -> np.ndarray:
    """fp16 bit patterns -> fp32 values (exact: every fp16 value is an fp32 value)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_bits(t) -> np.ndarray:
    """fp32 -> fp16 bit patterns by numpy's IEEE cast: round to nearest, ties to
    even, subnormal results kept, overflow to infinity."""
    with np.errstate(over="ignore"):          # overflow to infinity is the rule
        return np.asarray(t, dtype=np.float32).astype(np.float16).view(np.uint16)


_TO_F32 = {"bf16": bf16_bits_to_f32, "f16": f16_bits_to_f32}
_FROM_F32 = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}


def to_f32(bits, dtype: str = "bf16") -> np.ndarray:
    """16-bit input bit patterns of type dtype ('bf16' or 'f16') -> fp32."""
    return _TO_F32[dtype](bits)


def from_f32(t, dtype: str = "bf16") -> np.ndarray:
    """fp32 -> 16-bit output bit patterns of type dtype, round to nearest even."""
    return _FROM_F32[dtype](t)


# --- step 1/2: symmetric per-row int8 quantisation -----------------------

def quant_rows(rows_f32) -> tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 quantisation: returns (q int8 [R,K], scale fp32 [R]).

    Issue 5 probe, "Round two": dynamic per-token symmetric int8 activations;
    the same per-row maths gives the per-output-channel weight quantisation
    with fp32 scales (same section, artifact description).
    """
    a = np.asarray(rows_f32, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("rows must be 2-D")
    R, K = a.shape
    q = np.zeros((R, K), dtype=np.int8)
    if K == 0:
        return q, np.zeros(R, dtype=np.float32)
    amax = np.max(np.abs(a), axis=1)                      # exact
    scale = (amax / _F32_127).astype(np.float32)          # one fp32 division
    nz = scale != 0
    if np.any(nz):
        quot = a[nz] / scale[nz][:, None]                 # fp32 division
        assert quot.dtype == np.float32
        q[nz] = np.clip(np.rint(quot), -127, 127).astype(np.int8)  # RNE
    return q, scale


def quant_act(x_bits, dtype: str = "bf16") -> tuple[np.ndarray, np.ndarray]:
    """Dynamic per-token quantisation of bf16 (or fp16) activations [M,K]."""
    return quant_rows(to_f32(x_bits, dtype))


def quantize_weights(w_bits, dtype: str = "bf16") -> tuple[np.ndarray, np.ndarray]:
    """Load-time per-output-channel quantisation of bf16 (or fp16) weights
    [N,K] (Int8 Quantization guide, "Overview": quantise bf16 and fp16 weights at
    load).
    """
    return quant_rows(to_f32(w_bits, dtype))


# --- step 3: int8 x int8 -> int32 ----------------------------------------

def _check_k(K: int) -> None:
    if K > K_MAX:
        raise ValueError(f"K={K} exceeds {K_MAX}: int32 accumulation could overflow")


def gemm_exact(q, wq) -> np.ndarray:
    """acc[m,n] = sum_k q[m,k] * wq[n,k], exact, as int32.

    Computed with float64 BLAS on the int8-valued operands: every product and
    every partial sum is an integer of magnitude <= 127^2 K < 2^53, so any
    summation order gives the exact sum.
    """
    q = np.asarray(q, dtype=np.int8)
    wq = np.asarray(wq, dtype=np.int8)
    if q.shape[1] != wq.shape[1]:
        raise ValueError("K mismatch")
    _check_k(q.shape[1])
    acc = q.astype(np.float64) @ wq.astype(np.float64).T
    return acc.astype(np.int64).astype(np.int32)


def gemm_int64_rows(q, wq, rows=None) -> np.ndarray:
    """The same sum with literal int64 integer arithmetic, for chosen rows."""
    q = np.asarray(q, dtype=np.int8)
    wq64 = np.asarray(wq, dtype=np.int8).astype(np.int64)
    _check_k(q.shape[1])
    idx = range(q.shape[0]) if rows is None else rows
    out = [wq64 @ q[m].astype(np.int64) for m in idx]
    if not out:
        return np.zeros((0, wq64.shape[0]), dtype=np.int64)
    return np.stack(out)


# --- step 4: epilogue ----------------------------------------------------

def epilogue_f32(acc, s_a, s_w, bias_bits=None, dtype: str = "bf16") -> np.ndarray:
    """fp32 value before the output cast: ((fl32(acc) * s_a) * s_w) + bias.

    Issue 5 probe, "Round two": the result must carry act_scale (and the
    per-channel weight scale). Each operation rounds to fp32 separately. The
    bias has the output type dtype.
    """
    t = np.asarray(acc, dtype=np.int32).astype(np.float32)   # RNE beyond 2^24
    t = t * np.asarray(s_a, dtype=np.float32)[:, None]
    t = t * np.asarray(s_w, dtype=np.float32)[None, :]
    if bias_bits is not None:
        t = t + to_f32(bias_bits, dtype)[None, :]
    assert t.dtype == np.float32
    return t


def epilogue(acc, s_a, s_w, bias_bits=None, dtype: str = "bf16") -> np.ndarray:
    """Output bits (bf16 or fp16) of the epilogue."""
    return from_f32(epilogue_f32(acc, s_a, s_w, bias_bits, dtype), dtype)


# --- whole layer ---------------------------------------------------------

def linear(x_bits, wq, s_w, bias_bits=None, dtype: str = "bf16") -> dict:
    """W8A8 linear of x [M,K] (bf16, or fp16 with dtype='f16') with prepared
    int8 weights [N,K], fp32 s_w; bias and y have the type of x.

    Returns xq, s_a, acc (int32) and y (16-bit bits) so every intermediate
    can be compared.
    """
    xq, s_a = quant_act(x_bits, dtype)
    acc = gemm_exact(xq, wq)
    y = epilogue(acc, s_a, s_w, bias_bits, dtype)
    return {"xq": xq, "s_a": s_a, "acc": acc, "y": y}


# --- references the pages compare against -------------------------------

def dequant_reference(xq, s_a, wq, s_w, bias_bits=None) -> np.ndarray:
    """float64 (xq * s_a) @ (wq * s_w)^T (+ bias): the layer on its own
    quantised operands, which is what the Issue 5 probe compared the int8 ops
    against ("Kernel isolation": float32 x @ dequant(W)^T, with act_scale).
    """
    a = np.asarray(xq, np.float64) * np.asarray(s_a, np.float64)[:, None]
    b = np.asarray(wq, np.float64) * np.asarray(s_w, np.float64)[:, None]
    r = a @ b.T
    if bias_bits is not None:
        r = r + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return r


def float_reference(x_bits, w_bits, bias_bits=None) -> np.ndarray:
    """Unquantised float64 x @ W^T (+ bias)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    r = x @ w.T
    if bias_bits is not None:
        r = r + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return r


def noise_model_rel_l2(x_bits, w_bits, xq, s_a, wq, s_w) -> float:
    """Predicted rel-L2 of the quantised layer against the unquantised one.

    With independent, zero-mean rounding errors e_x (activations) and e_w
    (weights), E||(x+e_x)(W+e_w)^T - xW^T||^2 ~= sum e_x^2 (W^2)^T +
    sum x^2 (e_w^2)^T (the e_x e_w term is second order).
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    ex = np.asarray(xq, np.float64) * np.asarray(s_a, np.float64)[:, None] - x
    ew = np.asarray(wq, np.float64) * np.asarray(s_w, np.float64)[:, None] - w
    var = (ex**2 @ (w**2).T).sum() + (x**2 @ (ew**2).T).sum()
    ref = x @ w.T
    return float(np.sqrt(var) / np.linalg.norm(ref))


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


# --------------------------------------------------------------------------
# compressed-tensors pack-quantized ingest
#
# "Issue 5 probe ...", section "Round one: int8 weight-only via
# compressed-tensors": the int8 weight-only checkpoint stores its weights with
# compressed-tensors' pack_to_int32, as unsigned bytes offset by 128, four to a 32-bit word,
# with a per-output-channel scale.
# Readings where the page is silent: element 4i+j of a row sits in bits
# 8j..8j+7 of word i (little-endian, first element in the low byte); the int8
# value is the stored byte minus 128; the scale converts to fp32 exactly from
# fp32, bf16 or fp16.

def unpack_pack_quantized(packed_words) -> np.ndarray:
    """int32 words [N, W] -> int8 [N, 4W]: q[n, 4i+j] = ((word >> 8j) & 0xFF) - 128."""
    w = np.asarray(packed_words).astype(np.int64) & 0xFFFFFFFF
    N, W = w.shape
    q = np.empty((N, 4 * W), np.int16)
    for j in range(4):
        q[:, j::4] = ((w >> (8 * j)) & 0xFF) - 128
    return q.astype(np.int8)


def scale_to_f32(scale, dtype: str) -> np.ndarray:
    """Per-channel scale as fp32: dtype 'f32' (values), 'bf16' or 'f16' (bit patterns)."""
    a = np.asarray(scale)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(a.astype(np.uint16))
    if dtype == "f16":
        return a.astype(np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# W8A16: int8 weight-only with bf16 (or fp16) activations
#
# "Issue 5 probe ...", section "Round one: int8 weight-only via
# compressed-tensors": int8 weight-only (W8A16), per-output-channel symmetric
# weights, bf16 activations (no activation quantisation); the round's
# per-layer table runs the layers with bf16 and with fp16 activations.
# Readings where the page is silent: the per-channel scale is applied once
# to the sum, acc = sum_k fp32(x[k]) * wq[n,k] (each product is exact in
# fp32: 8 (bf16) or 11 (fp16) x 8 significant bits), y =
# round_to_nearest_even(fl32(fl32(acc) * s_w) + fp32(bias)) in the type of x;
# the oracle takes acc in float64 and rounds it to fp32 once. A kernel that
# accumulates in fp32 differs from it by its accumulation error, bounded in
# the parity test by a multiple of 2^-24 * sum_k |x[k] * wq[n,k]|.

def w8a16_acc(x_bits, wq, dtype: str = "bf16") -> np.ndarray:
    """float64 sum_k x[m,k] * wq[n,k] for x [M,K] (bf16 or fp16 bits) and int8 wq [N,K]."""
    x = to_f32(x_bits, dtype).astype(np.float64)
    return x @ np.asarray(wq, np.float64).T


def w8a16_abs_sum(x_bits, wq, dtype: str = "bf16") -> np.ndarray:
    """sum_k |x[m,k] * wq[n,k]|, the scale of the accumulation error."""
    x = np.abs(to_f32(x_bits, dtype).astype(np.float64))
    return x @ np.abs(np.asarray(wq, np.float64)).T


def w8a16_err_bound(x_bits, wq, s_w, dtype: str = "bf16") -> np.ndarray:
    """Bound on |t_kernel - t| for t = fl32(fl32(acc) * s_w) (+ bias), where
    the kernel accumulates acc in fp32 and this oracle rounds the exact sum
    once. Reading of the accumulation (the page names the scheme, not its
    arithmetic): two fp32 accumulators per output (the even and the odd
    16-element chunks of K) each take 2 * ceil(K / 128) additions of a
    32-product partial dot, and one addition joins them, so a product meets
    n = 2 * ceil(K / 128) + 1 sequential roundings after its partial dot; the
    partial dot of 32 exact products rounds each of them at most 8 times. The
    standard summation bound then gives gamma_{n+8} * sum|x * wq| with
    gamma_j ~ j * 2^-24; (2n + 8) * 2^-24 * sum|x * wq| also covers the
    oracle's own rounding of the exact sum to fp32, and the bound scales with
    |s_w| through the (monotone) fp32 product. A parity test adds one unit in
    the last place of the output type, where a rounding boundary may fall
    between the two values."""
    K = np.asarray(x_bits).shape[1]
    n = 2 * ((K + 127) // 128) + 1
    return (2 * n + 8) * 2.0**-24 * w8a16_abs_sum(x_bits, wq, dtype) * np.abs(
        np.asarray(s_w, np.float64))[None, :]


def w8a16_linear(x_bits, wq, s_w, bias_bits=None, dtype: str = "bf16") -> dict:
    """W8A16 linear: x [M,K] (bf16, or fp16 with dtype='f16'), int8 wq [N,K],
    fp32 s_w [N] -> y bits of the type of x (bias has that type too).

    Returns acc (float64) and y.
    """
    acc = w8a16_acc(x_bits, wq, dtype)
    t = acc.astype(np.float32)                                   # one RNE rounding
    t = t * np.asarray(s_w, dtype=np.float32)[None, :]
    if bias_bits is not None:
        t = t + to_f32(bias_bits, dtype)[None, :]
    assert t.dtype == np.float32
    return {"acc": acc, "y": from_f32(t, dtype)}


# --------------------------------------------------------------------------
# Producer fusion: the normalisation and the activation that produce a
# linear's input, writing its int8 codes and per-row scales directly
#
# "Qwen-Image-2.1: TE AutoRound-AWQ on GPU + all-resident single-3090 stack",
# section "Whole-pipeline follow-up": the W8A8 DiT path's kernel trace holds
# the int8 GEMMs plus fused activation-quantisation, normalisation and
# activation kernels around them. The page names those kernels, not their
# formulas. Readings taken here:
#
# * the normalisation is the adaptive (modulated) LayerNorm in front of a DiT
#   block's QKV and FFN-up linears: per row, the mean and the biased variance
#   over K, then v = (x - mean) / sqrt(var + eps) * (1 + scale) + shift, with
#   shift and scale bf16 vectors [K] shared by a group of rows (the tokens of
#   one sample) and no learnt affine of its own;
# * the activation is GELU in front of FFN-down: z * Phi(z), Phi the standard
#   normal distribution function ("erf" form), or its tanh approximation
#   0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)));
# * the fused kernel computes what the unfused producer would write, v
#   rounded to bf16 (nearest, ties to even), and quantises that bf16 row
#   exactly as quant_act does.
#
# The oracle takes v in float64 and rounds it to bf16 once. A kernel that
# evaluates v in fp32 is off by its rounding error; the *_err_bound functions
# bound that error, and the parity tests allow it on top of bf16's own half
# ulp. The int8 codes and scales are compared bit for bit after quantising
# the kernel's own bf16 row, so both sides take the integer decisions on the
# same bf16 values.

def f64_to_bf16_bits(v) -> np.ndarray:
    """float64 -> bf16 bit patterns with a single round to nearest even.

    Rounding to fp32 first and then to bf16 can round twice the wrong way (a
    value just above a bf16 midpoint can land on it in fp32). The first step
    therefore rounds to odd: truncate toward zero to fp32, then set the last
    bit if anything was dropped. With 16 more bits than bf16 that keeps every
    later tie decision exact. Subnormals are kept; past the bf16 range the
    result is infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    back = f.astype(np.float64)
    bits = f.view(np.uint32).copy()
    inexact = back != v
    # magnitude one fp32 step toward zero where the nearest rounding went up
    # (sign-magnitude patterns: decrementing the pattern shrinks |f|)
    bits[inexact & (np.abs(back) > np.abs(v))] -= np.uint32(1)
    bits[inexact] |= np.uint32(1)
    return f32_to_bf16_bits(bits.view(np.float32))


def _mod_rows(M: int, rows_per_group):
    rpg = M if rows_per_group is None else int(rows_per_group)
    if rpg < 1:
        raise ValueError("rows_per_group must be >= 1")
    return np.arange(M) // rpg


def layernorm_modulate(x_bits, shift_bits, scale_bits, eps: float, rows_per_group=None):
    """float64 v [M,K] of the modulated LayerNorm of bf16 rows x [M,K].

    shift, scale: bf16 [G,K]; row m uses group m // rows_per_group (one
    group for all rows when rows_per_group is None). eps is taken as the
    fp32 value the kernel receives.
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    M, K = x.shape
    g = _mod_rows(M, rows_per_group)
    sh = bf16_bits_to_f32(np.atleast_2d(shift_bits)).astype(np.float64)
    sc = bf16_bits_to_f32(np.atleast_2d(scale_bits)).astype(np.float64)
    mean = x.mean(axis=1, keepdims=True)
    d = x - mean
    var = (d * d).mean(axis=1, keepdims=True)
    e = float(np.float32(eps))
    with np.errstate(divide="ignore", invalid="ignore"):
        return d / np.sqrt(var + e) * (1.0 + sc[g]) + sh[g]


def gelu(z_bits, approximate: str = "none") -> np.ndarray:
    """float64 GELU of bf16 z: z * Phi(z) ('none') or the tanh form ('tanh').

    Phi(z) = erfc(-z / sqrt 2) / 2 (no cancellation for z << 0). The tanh
    form is evaluated through 0.5 (1 + tanh t) = 1 / (1 + exp(-2t)), which
    is the same function without the cancellation of 1 + tanh(t) at t << 0.
    """
    from scipy.special import erfc
    z = bf16_bits_to_f32(z_bits).astype(np.float64)
    if approximate == "none":
        return 0.5 * z * erfc(-z / np.sqrt(2.0))
    if approximate == "tanh":
        t = np.sqrt(2.0 / np.pi) * (z + 0.044715 * z * z * z)
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-2.0 * t))
    raise ValueError(approximate)


def producer_quant(v) -> dict:
    """bf16 row values of the producer (nearest to v) and their quantisation."""
    y = f64_to_bf16_bits(v)
    xq, s = quant_act(y)
    return {"y": y, "xq": xq, "a_scale": s}


def layernorm_modulate_quant(x_bits, shift_bits, scale_bits, eps: float,
                             rows_per_group=None) -> dict:
    return producer_quant(layernorm_modulate(x_bits, shift_bits, scale_bits, eps,
                                             rows_per_group))


def gelu_quant(z_bits, approximate: str = "none") -> dict:
    return producer_quant(gelu(z_bits, approximate))


_U32 = 2.0 ** -24


def layernorm_modulate_err_bound(x_bits, shift_bits, scale_bits, eps: float,
                                 rows_per_group=None, depth=None) -> np.ndarray:
    """Bound on |v32 - v| for an fp32 evaluation v32 of the modulated LayerNorm
    (u = 2^-24, first order, doubled). depth is the longest chain of fp32
    additions any term of the two row sums passes through: K - 1 when the
    order is unknown (the default), less for a blocked or tree reduction.

      mean:  |mean32 - mean| <= (depth + 1) u m1          (m1 = mean |x|)
      d = x - mean32: off by that plus u |d|
      var:   relative error <= (depth + 2) u, plus (mean32 - mean)^2 / var
      rstd = 1 / sqrt(var + eps): relative error <= (depth + 3) u / 2 + 2 u
      (1 + scale), the two products and the sum with shift: 4 u in all
    so |v32 - v| <= (depth + 1) u m1 rstd |g| + (depth / 2 + 8) u |A|
                    + u |shift| + (dm)^2 |A| / 2,
    with A = (x - mean) rstd g and dm = (depth + 1) u m1 rstd.
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    M, K = x.shape
    D = (K - 1) if depth is None else int(depth)
    g = _mod_rows(M, rows_per_group)
    sh = bf16_bits_to_f32(np.atleast_2d(shift_bits)).astype(np.float64)[g]
    gain = 1.0 + bf16_bits_to_f32(np.atleast_2d(scale_bits)).astype(np.float64)[g]
    mean = x.mean(axis=1, keepdims=True)
    d = x - mean
    rstd = 1.0 / np.sqrt((d * d).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    m1 = np.abs(x).mean(axis=1, keepdims=True)
    a = np.abs(d * rstd * gain)
    dm = (D + 1) * _U32 * m1 * rstd
    e = dm * np.abs(gain) + (D / 2 + 8) * _U32 * a + _U32 * np.abs(sh) + 0.5 * dm * dm * a
    return 2.0 * e + 2.0 ** -145


def gelu_err_bound(z_bits, approximate: str = "none") -> np.ndarray:
    """Bound on |v32 - v| for an fp32 evaluation of GELU by the forms above with
    the fp32 library erfc / exp (each within 16 u of its result), doubled:

      'none': the argument a = z / sqrt 2 carries 2 u, which erfc magnifies
              by its condition number, at most 3 a^2 + 2; the library 16 u;
              the two products 2 u:  (6 a^2 + 22) u |v|.
      'tanh': t = sqrt(2/pi) (z + 0.044715 z^3) carries 8 u, e = exp(-2|t|)
              magnifies it by 2|t|; the library 16 u; 1 + e and the
              division 2 u:  (16 |t| + 20) u |v|. (An fp32 evaluation takes
              z / (1 + e) for t >= 0 and z e / (1 + e) for t < 0: exp(-2t)
              itself overflows for t < -44 while v is still an fp32 normal.)
    Plus 2^-144 for results and intermediates in the fp32 subnormal range.
    """
    z = bf16_bits_to_f32(z_bits).astype(np.float64)
    v = np.abs(gelu(z_bits, approximate))
    if approximate == "none":
        a = z / np.sqrt(2.0)
        rel = (6.0 * a * a + 22.0) * _U32
    elif approximate == "tanh":
        t = np.sqrt(2.0 / np.pi) * (z + 0.044715 * z * z * z)
        rel = (16.0 * np.abs(t) + 20.0) * _U32
    else:
        raise ValueError(approximate)
    return 2.0 * rel * v + 2.0 ** -144


def bf16_within(y_bits, v, err) -> np.ndarray:
    """True where the bf16 value y is a correct result for the exact v when
    the evaluation may be off by err: |y - v| <= half a bf16 ulp at v + err
    (at a binade edge, half an ulp of the binade below). Infinite y is
    accepted only where v is past the bf16 overflow threshold."""
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    v = np.asarray(v, np.float64)
    av = np.abs(v)
    e = np.frexp(np.maximum(av, 2.0 ** -126))[1] - 1         # exact binade of |v|
    half_ulp = np.ldexp(1.0, e - 8)
    ok = np.abs(y - v) <= half_ulp + err
    big = av + err >= (2.0 - 2.0 ** -8) * 2.0 ** 127
    return np.where(np.isinf(y), big & (np.sign(y) == np.sign(v)), ok)
