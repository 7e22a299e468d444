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


# --- the accumulation error bound of the parity tests ------------------------

def _ulp(v, dtype="bf16"):
    v = np.abs(np.asarray(v, np.float64))
    bits, tiny = (7, -133) if dtype == "bf16" else (10, -24)
    e = np.floor(np.log2(np.maximum(v, 2.0**tiny)))
    return np.maximum(2.0 ** (e - bits), 2.0**tiny)


def _fp32_kernel_order(x_bits, wq, sw, bias_bits=None, inner="tree", mistake=None):
    """An fp32 evaluation with the accumulation structure the bound assumes:
    two accumulators (even / odd 16-element chunks of K), each adding a
    32-product partial dot per step in K order, joined by one final addition.
    inner: how a partial dot sums its 32 exact products ("tree": pairwise,
    "seq4": runs of 4 then pairwise). mistake: a plausible kernel defect."""
    x = oracle.bf16_bits_to_f32(x_bits)
    M, K = x.shape
    N = wq.shape[0]
    Kp = (K + 127) // 128 * 128
    xp = np.zeros((M, Kp), np.float32)
    xp[:, :K] = x
    wp = np.zeros((N, Kp), np.float32)
    wp[:, :K] = wq
    if mistake == "drop_last_window":
        wp[:, Kp - 128:] = 0
    prods = xp[:, None, :] * wp[None, :, :]                      # exact in fp32
    chunks = prods.reshape(M, N, Kp // 16, 16)
    accs = []
    for parity in (0, 1):
        part = chunks[:, :, parity::2, :].reshape(M, N, Kp // 64, 32)
        if inner == "seq4":
            part = np.add.accumulate(part.reshape(M, N, Kp // 64, 8, 4), axis=-1,
                                     dtype=np.float32)[..., -1]
        while part.shape[-1] > 1:
            part = part[..., 0::2] + part[..., 1::2]
        part = part[..., 0]
        acc = np.zeros((M, N), np.float32)
        for step in range(part.shape[-1]):
            p = part[..., step]
            if mistake == "bf16_partials":
                p = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(p))
            acc = acc + p
            if mistake == "bf16_accumulator":
                acc = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(acc))
        accs.append(acc)
    acc = accs[0] if mistake == "no_pair_sum" else accs[0] + accs[1]
    s = np.asarray(sw, np.float32)
    if mistake == "shifted_scale":
        s = np.roll(s, 1)
    t = acc * s[None, :]
    if bias_bits is not None:
        t = t + oracle.bf16_bits_to_f32(bias_bits)[None, :]
    return oracle.f32_to_bf16_bits(t)


def _bound_case(kind, M=3, K=8064, N=24, seed=0):
    rng = np.random.default_rng(500 + seed)
    if kind == "random":
        x = random_bf16(rng, (M, K), 1.0)
        wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    elif kind == "positive":          # every product positive: the rounding errors add up
        x = to_bf16(np.abs(rng.standard_normal((M, K))) + 0.5)
        wq = rng.integers(64, 128, (N, K)).astype(np.int8)
    else:                             # mixed magnitudes across K
        mag = np.where(rng.random(K) < 0.05, 1000.0, np.where(rng.random(K) < 0.5, 1e-3, 1.0))
        x = to_bf16(rng.standard_normal((M, K)) * mag[None, :])
        wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    bias = random_bf16(rng, (N,), 0.01)
    return x, wq, sw, bias


def _violations(x, wq, sw, bias, y_bits):
    ye = oracle.w8a16_linear(x, wq, sw, bias)["y"]
    y = oracle.bf16_bits_to_f32(y_bits).astype(np.float64)
    yv = oracle.bf16_bits_to_f32(ye).astype(np.float64)
    tol = oracle.w8a16_err_bound(x, wq, sw) + _ulp(np.maximum(np.abs(y), np.abs(yv)))
    return np.abs(y - yv) > tol


@pytest.mark.parametrize("kind", ["random", "positive", "mixed"])
@pytest.mark.parametrize("inner", ["tree", "seq4"])
def test_w8a16_bound_holds_for_the_kernel_structure(kind, inner):
    """The parity bar (bound + 1 ulp) accepts fp32 accumulation in the
    structure it was derived for, including inputs whose rounding errors all
    have the same sign, at the largest K the kernel takes (8064)."""
    x, wq, sw, bias = _bound_case(kind)
    assert not _violations(x, wq, sw, bias, _fp32_kernel_order(x, wq, sw, bias, inner)).any()


@pytest.mark.parametrize("mistake", ["bf16_accumulator", "bf16_partials", "drop_last_window",
                                     "no_pair_sum", "shifted_scale"])
def test_w8a16_bound_rejects_plausible_mistakes(mistake):
    """The bar is tight enough to catch kernel defects on the modulation
    projection's shape class (K = 3072, Gaussian activations)."""
    x, wq, sw, bias = _bound_case("random", M=2, K=3072, N=64, seed=1)
    bad = _fp32_kernel_order(x, wq, sw, bias, "tree", mistake)
    assert _violations(x, wq, sw, bias, bad).mean() > 0.05


def test_w8a16_bound_against_output_ulp():
    """On Gaussian inputs at K = 3072 the accumulation bound is a fraction of
    the output ulp, so the bar accepts the other bf16 neighbour of the exact
    value only near rounding midpoints."""
    x, wq, sw, bias = _bound_case("random", M=4, K=3072, N=256, seed=2)
    ye = oracle.w8a16_linear(x, wq, sw, bias)["y"]
    ratio = oracle.w8a16_err_bound(x, wq, sw) / _ulp(oracle.bf16_bits_to_f32(ye))
    assert np.median(ratio) < 0.25
