"""Pins of the oracle's per-row symmetric int8 quantisation (CPU only).

Each test checks the oracle against something other than itself: hand
values, exact rational arithmetic written from the IEEE definition, a
theorem-backed float64 route, or invariants of the definition.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_arith import f32_div, round_half_even
from golden_io import quant_cases
from synth_inputs import all_finite_bf16, to_bf16_bits


def _bits(vals):
    # values in the golden files are exact in bf16; check that they are
    f = np.asarray(vals, dtype=np.float64)
    b = to_bf16_bits(f)
    assert np.array_equal(oracle.bf16_bits_to_f32(b).astype(np.float64), f)
    return b


@pytest.mark.parametrize("case", quant_cases())
def test_quant_hand_cases(case):
    xs, s, qs = case
    q, scale = oracle.quant_act(_bits(xs)[None, :])
    assert scale[0] == np.float32(s)
    assert q[0].tolist() == qs


def _exact_quant_row(row_f32):
    """q and scale of one row by exact rationals (fp32 IEEE divisions)."""
    amax = max(abs(Fraction(float(v))) for v in row_f32)
    s = f32_div(float(amax), 127.0)
    if s == 0:
        return [0] * len(row_f32), 0.0
    q = []
    for v in row_f32:
        t = f32_div(float(v), float(s))
        q.append(max(-127, min(127, round_half_even(t))))
    return q, float(s)


def test_quant_exact_rational_random():
    rng = np.random.default_rng(1)
    rows = []
    # ordinary rows, heavy tails, and rows whose scale is an fp32 subnormal
    for j in range(24):
        r = rng.standard_normal(37) * (10.0 ** rng.uniform(-3, 3))
        if j % 4 == 1:
            r = rng.standard_t(2.0, 37)
        if j % 4 == 2:
            r = rng.standard_normal(37) * 2.0 ** -128
        if j % 4 == 3:
            r = rng.standard_normal(37) * 2.0 ** -131
        rows.append(r)
    x = np.stack([to_bf16_bits(r) for r in rows])
    q, s = oracle.quant_act(x)
    xf = oracle.bf16_bits_to_f32(x)
    for i in range(x.shape[0]):
        eq, es = _exact_quant_row(xf[i])
        assert float(s[i]) == es, i
        assert q[i].tolist() == eq, i
    # the subnormal-scale rows really had subnormal scales
    assert np.any((s > 0) & (s < np.finfo(np.float32).tiny))


def test_quant_division_not_reciprocal():
    """x/s and x*(1/s) differ on some bf16 values; the oracle must take x/s.

    Found by exact search over one amax; the expected q is the exact-rational
    fp32 quotient rounded half to even.
    """
    amax = 3.8125
    vals = oracle.bf16_bits_to_f32(all_finite_bf16())
    vals = vals[np.abs(vals) <= amax]
    row = np.concatenate([[amax], vals]).astype(np.float32)
    q, s = oracle.quant_rows(row[None, :])
    s = s[0]
    recip = np.float32(1.0) / s
    q_recip = np.clip(np.rint(row * recip), -127, 127)
    diff = np.nonzero(q_recip != q[0])[0]
    assert diff.size > 0          # the two forms do differ here
    for i in diff:
        t = f32_div(float(row[i]), float(s))
        assert q[0][i] == round_half_even(t)


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4074, 0x43E0, 0x007F, 0x0001,
                                       0x0080, 0x7F7F, 0x3C01, 0xC2FE])
def test_quant_exhaustive_bf16(amax_bits):
    """All finite bf16 values below one amax, against the float64 route.

    fl32(fl64(a/b)) equals the correctly rounded fp32 quotient of two fp32
    values because float64 carries more than 2*24+2 significant bits (double
    rounding is innocuous for division), so this is an independent exact
    reference for every element.
    """
    amax = float(oracle.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
    allv = oracle.bf16_bits_to_f32(all_finite_bf16())
    vals = allv[np.abs(allv) <= abs(amax)]
    row = np.concatenate([[amax], vals]).astype(np.float32)
    q, s = oracle.quant_rows(row[None, :])
    s64 = np.float32(np.float64(abs(amax)) / 127.0)
    assert s[0] == s64
    ref = np.rint((row.astype(np.float64) / np.float64(s64)).astype(np.float32))
    ref = np.clip(ref, -127, 127)
    assert np.array_equal(q[0].astype(np.float64), ref)
    assert np.abs(q[0]).max() == 127


def test_quant_clamp_never_needed_for_bf16():
    """For every finite bf16 amax, round(amax/scale) is exactly 127.

    So the [-127,127] clamp never engages for bf16 inputs, subnormal scales
    included (the smallest bf16 subnormal still gives a scale of 516 fp32
    subnormal quanta). Checked with exact rationals on the subnormal and
    lowest-normal amax values and with the float64 route on all of them.
    """
    allv = oracle.bf16_bits_to_f32(all_finite_bf16()).astype(np.float64)
    pos = allv[allv > 0]
    s = (pos / 127.0).astype(np.float32)
    t = (pos / s.astype(np.float64)).astype(np.float32)
    assert np.all(np.rint(t) == 127)
    for a in pos[:300]:
        sa = f32_div(float(a), 127.0)
        assert round_half_even(f32_div(float(a), float(sa))) == 127


def test_quant_invariants():
    rng = np.random.default_rng(2)
    x = to_bf16_bits(rng.standard_normal((16, 96)) * 3.0)
    q, s = oracle.quant_act(x)
    # symmetric: q(-x) = -q(x), same scale
    qn, sn = oracle.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # power-of-two scaling: x * 2^j gives s * 2^j and the same q
    for j in (-20, -3, 5, 40):
        xs = to_bf16_bits(oracle.bf16_bits_to_f32(x).astype(np.float64) * 2.0**j)
        qj, sj = oracle.quant_act(xs)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s.astype(np.float64) * 2.0**j).astype(np.float32))
    # every row with a normal scale reaches +-127; -128 never appears
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127
    # rows are independent of their neighbours and of M
    q1, s1 = oracle.quant_act(x[5:6])
    assert np.array_equal(q1[0], q[5]) and s1[0] == s[5]
    # RNE error bound: |x - q*s| <= s/2 up to the fp32 rounding of x/s
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    err = np.abs(xf - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0**-17))


def test_quant_zero_and_empty():
    q, s = oracle.quant_act(np.zeros((3, 8), np.uint16))
    assert np.all(q == 0) and np.all(s == 0)
    q, s = oracle.quant_act(np.zeros((0, 8), np.uint16))
    assert q.shape == (0, 8) and s.shape == (0,)


def test_quant_matches_symmetric_definition_on_weights():
    """Weights use the same per-row maths (one fp32 scale per output row)."""
    rng = np.random.default_rng(3)
    w = to_bf16_bits(rng.normal(0, 0.02, (9, 40)))
    qa, sa = oracle.quant_act(w)
    qw, sw = oracle.quantize_weights(w)
    assert np.array_equal(qa, qw) and np.array_equal(sa, sw)
    assert sw.dtype == np.float32


def test_bf16_decode_matches_torch():
    b = all_finite_bf16()
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_bits_to_f32(b).view(np.uint32), t.view(np.uint32))
