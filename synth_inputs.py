"""Seeded synthetic inputs for the W8A8 int8-dynamic linear layer.

This module only draws random tensors and stores them as bf16 bit patterns
(numpy uint16). It holds none of the layer's arithmetic (no quantisation, no
GEMM, no epilogue), so the CPU oracle and the HIP path can both take their
inputs from it without sharing any computation.

Recipe (the same for every workload):

* RNG: ``numpy.random.default_rng(seed)`` (PCG64), seed 0 unless stated.
* Values are drawn in float64, scaled, cast to float32 and then to bfloat16
  by torch-CPU (round to nearest even at both casts).
* Draw order: activation base values, then outlier channel indices
  (``rng.choice(K, round(p*K), replace=False)``), then the weight, then the
  bias.

Workloads stand in for the linears of a 1024px diffusion transformer
(hidden 3072, MLP 12288, 4096 image + 256 text tokens) and its AdaLN
modulation projection at batch 1, which the pages describe: Qwen-Image-2.1
whole-pipeline W8A8 DiT path (Qwen-Image-2.1 page, "Whole-pipeline follow-up")
and the int8 M=1 modulation crash (unsloth test_diffusion_transformer_quant.py
commit log). The first three shapes are the ones the Issue 5 probe
("Round two" section) checked its int8 ops on.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class LinearSpec:
    name: str
    M: int
    K: int
    N: int
    x_dist: str = "normal"        # normal | student_t4 | gelu_normal
    outlier_frac: float = 0.0     # fraction of input channels scaled
    outlier_gain: float = 1.0
    w_std: float = 0.02
    bias_std: float | None = None  # None: no bias
    seed: int = 0


def _spec_table():
    specs = [
        LinearSpec("c1_64x256x128", 64, 256, 128, bias_std=0.01),
        LinearSpec("c2_512x4096x4096_outliers", 512, 4096, 4096,
                   outlier_frac=0.01, outlier_gain=20.0),
        LinearSpec("c3_512x4096x12288_student_t", 512, 4096, 12288,
                   x_dist="student_t4", bias_std=0.01),
        LinearSpec("dit_qkv_4352x3072x9216", 4352, 3072, 9216,
                   outlier_frac=0.005, outlier_gain=30.0),
        LinearSpec("dit_out_4352x3072x3072", 4352, 3072, 3072,
                   outlier_frac=0.005, outlier_gain=30.0),
        LinearSpec("dit_up_4352x3072x12288", 4352, 3072, 12288,
                   outlier_frac=0.005, outlier_gain=30.0),
        LinearSpec("dit_down_4352x12288x3072", 4352, 12288, 3072,
                   x_dist="gelu_normal", outlier_frac=0.005, outlier_gain=30.0),
    ]
    for m in (1, 2, 8, 16, 17, 32):
        specs.append(LinearSpec(f"mod_m{m}_3072x18432", m, 3072, 18432,
                                bias_std=0.01))
    return {s.name: s for s in specs}


SPECS = _spec_table()

# The four block linears of one 1024px DiT block plus its modulation
# projection at batch 1: one pass over these is one step of the benchmark.
DIT_BLOCK = ("dit_qkv_4352x3072x9216", "dit_out_4352x3072x3072",
             "dit_up_4352x3072x12288", "dit_down_4352x12288x3072",
             "mod_m1_3072x18432")


def to_bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> bfloat16 bit patterns (uint16), RNE casts."""
    f32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def draw_x(rng: np.random.Generator, spec: LinearSpec, M: int | None = None) -> np.ndarray:
    M = spec.M if M is None else M
    K = spec.K
    if spec.x_dist == "normal":
        x = rng.standard_normal((M, K))
    elif spec.x_dist == "student_t4":
        x = rng.standard_t(4.0, size=(M, K))
    elif spec.x_dist == "gelu_normal":
        x = _gelu_erf(rng.standard_normal((M, K)))
    else:
        raise ValueError(spec.x_dist)
    if spec.outlier_frac > 0:
        n_out = int(round(spec.outlier_frac * K))
        cols = rng.choice(K, n_out, replace=False)
        x[:, cols] *= spec.outlier_gain
    return x


def make_linear_inputs(spec: LinearSpec | str, M: int | None = None) -> dict:
    """Inputs of one linear: x [M,K], w [N,K], bias [N] or None (bf16 bits)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    rng = np.random.default_rng(spec.seed)
    x = to_bf16_bits(draw_x(rng, spec, M))
    w = to_bf16_bits(rng.normal(0.0, spec.w_std, size=(spec.N, spec.K)))
    bias = None
    if spec.bias_std is not None:
        bias = to_bf16_bits(rng.normal(0.0, spec.bias_std, size=(spec.N,)))
    return {"name": spec.name, "M": x.shape[0], "K": spec.K, "N": spec.N,
            "x": x, "w": w, "bias": bias}


def to_f16_bits(a) -> np.ndarray:
    """float64/float32 array -> IEEE fp16 bit patterns (uint16), RNE casts via
    fp32 (numpy's cast; values past 65504 become infinity)."""
    f32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    with np.errstate(over="ignore"):
        return f32.astype(np.float16).view(np.uint16).copy()


def random_f16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std^2) fp16 bits, for the fp16 parity cases."""
    return to_f16_bits(rng.normal(0.0, std, size=shape))


def all_finite_f16() -> np.ndarray:
    """Every finite fp16 bit pattern (both zeros included): 63 488 values."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return bits[((bits >> 10) & 0x1F) != 0x1F]


def random_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std^2) bf16 bits, for small parity cases of any shape."""
    return to_bf16_bits(rng.normal(0.0, std, size=shape))


def all_finite_bf16() -> np.ndarray:
    """Every finite bf16 bit pattern (both zeros included): 65 280 values."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]
