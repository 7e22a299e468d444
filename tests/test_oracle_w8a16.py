"""Pins of the oracle's W8A16 (int8 weight-only, bf16 activations) linear,
CPU only: hand-computed outputs, the exact rational sum and fp32/bf16
roundings written from their definitions, a closed form, and agreement with
the float64 dequantised-weight product (scale per output channel)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_arith import f32_add, f32_mul, to_bf16_bits, to_f32
from golden_io import w8a16_cases
from synth_inputs import random_bf16, to_bf16_bits as to_bf16


def _bits(vals):
    return to_bf16(np.asarray(vals, np.float64))


def test_hand_computed_cases():
    cases = w8a16_cases()
    assert len(cases) >= 6
    for xs, ws, s, b, y in cases:
        x = _bits(xs)[None, :]
        assert np.array_equal(oracle.bf16_bits_to_f32(x)[0], np.asarray(xs, np.float32))
        bias = None if b is None else np.array([b], np.uint16)
        got = oracle.w8a16_linear(x, np.array([ws], np.int8), np.array([s], np.float32), bias)
        assert int(got["y"][0, 0]) == y, (xs, ws, s, b, hex(int(got["y"][0, 0])), hex(y))


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_reference(seed):
    """acc is the exact sum; y the fp32 / bf16 roundings from their definitions."""
    rng = np.random.default_rng(seed)
    M, K, N = 2, 24, 3
    x = random_bf16(rng, (M, K), 1.0 if seed % 2 else 1e-3)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-3, 1e-1, N).astype(np.float32)
    bias = random_bf16(rng, (N,), 0.1) if seed % 3 == 0 else None
    got = oracle.w8a16_linear(x, wq, sw, bias)
    xf = oracle.bf16_bits_to_f32(x)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * int(wq[n, k]) for k in range(K))
            assert Fraction(float(got["acc"][m, n])) == exact
            t = f32_mul(float(to_f32(exact)), float(sw[n]))
            if bias is not None:
                t = f32_add(float(t), float(oracle.bf16_bits_to_f32(bias)[n]))
            assert int(got["y"][m, n]) == to_bf16_bits(t)


def test_closed_form_all_max_weights():
    K = 64
    x = np.full((1, K), 0x3F80, np.uint16)                  # 1.0
    wq = np.full((2, K), 127, np.int8)
    wq[1] = -127
    got = oracle.w8a16_linear(x, wq, np.array([1.0, 0.5], np.float32))
    assert got["acc"].tolist() == [[127.0 * K, -127.0 * K]]
    assert oracle.bf16_bits_to_f32(got["y"]).tolist() == [[127.0 * K, -63.5 * K]]


def test_matches_dequantised_weight_product():
    """sum_k x (wq * s_w) in float64 agrees to within a bf16 ulp: the scale
    belongs to the output channel (a transposed or per-input scale fails)."""
    rng = np.random.default_rng(9)
    M, K, N = 4, 256, 40
    x = random_bf16(rng, (M, K))
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    y = oracle.bf16_bits_to_f32(oracle.w8a16_linear(x, wq, sw)["y"]).astype(np.float64)
    ref = oracle.bf16_bits_to_f32(x).astype(np.float64) @ (wq.astype(np.float64) * sw[:, None]).T
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2.0**-8 + 1e-30)


# ---- fp16 activations (the probe's Round one ran bf16 and fp16 acts) -------

def test_f16_hand_computed_cases():
    from synth_inputs import to_f16_bits
    cases = w8a16_cases("w8a16_f16_hand_cases.txt")
    assert len(cases) >= 5
    for xs, ws, s, b, y in cases:
        x = to_f16_bits(np.asarray(xs, np.float64))[None, :]
        assert np.array_equal(oracle.f16_bits_to_f32(x)[0], np.asarray(xs, np.float32))
        bias = None if b is None else np.array([b], np.uint16)
        got = oracle.w8a16_linear(x, np.array([ws], np.int8), np.array([s], np.float32), bias,
                                  "f16")
        assert int(got["y"][0, 0]) == y, (xs, ws, s, b, hex(int(got["y"][0, 0])), hex(y))


@pytest.mark.parametrize("seed", range(4))
def test_f16_exact_rational_reference(seed):
    """fp16 x: acc is the exact sum, y the fp32 / fp16 roundings from their
    definitions (exact_arith.to_f16_bits)."""
    from exact_arith import to_f16_bits as exact_f16
    from synth_inputs import random_f16
    rng = np.random.default_rng(100 + seed)
    M, K, N = 2, 24, 3
    x = random_f16(rng, (M, K), 1.0 if seed % 2 else 1e-3)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-3, 1e-1, N).astype(np.float32)
    bias = random_f16(rng, (N,), 0.1) if seed % 2 == 0 else None
    got = oracle.w8a16_linear(x, wq, sw, bias, "f16")
    xf = oracle.f16_bits_to_f32(x)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * int(wq[n, k]) for k in range(K))
            assert Fraction(float(got["acc"][m, n])) == exact
            t = f32_mul(float(to_f32(exact)), float(sw[n]))
            if bias is not None:
                t = f32_add(float(t), float(oracle.f16_bits_to_f32(bias)[n]))
            assert int(got["y"][m, n]) == exact_f16(t)
