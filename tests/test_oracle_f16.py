"""Pins of the oracle's fp16 activation/output variant (CPU only).

The fp16 variant is the W8A8 layer with fp16 in place of bf16 for x, W, bias
and y ("Int8 Quantization" guide, "Overview": BF16/FP16 weights; Issue 5
probe, "Round one": bf16 and fp16 activations). Each test checks the oracle
against something other than itself: the binary16 definition, hand values
(tests/golden/f16_hand_cases.txt), exact rational arithmetic, a
theorem-backed float64 route, the bf16 path on values both formats hold, and
the float64 dequantised reference.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_arith import f32_add, f32_mul, round_half_even, to_f16_bits, f32_div
from golden_io import f16_cases
from synth_inputs import to_bf16_bits

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[((ALL >> 10) & 0x1F) != 0x1F]


def _f16_value(b: int) -> Fraction:
    """binary16 pattern -> exact value, from the format's definition."""
    s, e, m = b >> 15, (b >> 10) & 0x1F, b & 0x3FF
    v = Fraction(m, 1024) * Fraction(2) ** -14 if e == 0 else \
        (1 + Fraction(m, 1024)) * Fraction(2) ** (e - 15)
    return -v if s else v


def _bits(vals):
    b = oracle.f32_to_f16_bits(np.asarray(vals, np.float64).astype(np.float32))
    assert np.array_equal(oracle.f16_bits_to_f32(b).astype(np.float64), np.asarray(vals, np.float64))
    return b


def test_f16_decode_definition():
    got = oracle.f16_bits_to_f32(FINITE).astype(np.float64)
    ref = np.array([float(_f16_value(int(b))) for b in FINITE])
    assert np.array_equal(got, ref)
    inf = oracle.f16_bits_to_f32(np.array([0x7C00, 0xFC00], np.uint16))
    assert inf[0] == np.inf and inf[1] == -np.inf


def test_f16_round_midpoints_exhaustive():
    """Every midpoint between neighbouring fp16 values (exact in fp32) goes to
    the even neighbour; the fp32 values next to it go to the near side. The
    top pair is (65504, infinity), with midpoint 65520."""
    pos = FINITE[FINITE < 0x8000].astype(np.int64)
    pos = np.sort(pos)
    a = oracle.f16_bits_to_f32(pos.astype(np.uint16)).astype(np.float64)
    b = np.append(a[1:], 65536.0)            # the next value up (65536 stands in for inf)
    nb = np.append(pos[1:], 0x7C00)
    mid = ((a + b) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (a + b) / 2)   # exact in fp32
    even = np.where(pos % 2 == 0, pos, nb)
    for sign in (1, -1):
        sb = 0 if sign > 0 else 0x8000
        got = oracle.f32_to_f16_bits(sign * mid).astype(np.int64)
        assert np.array_equal(got, even | sb)
        up = np.nextafter(sign * mid, np.float32(sign * np.inf))
        dn = np.nextafter(sign * mid, np.float32(0))
        assert np.array_equal(oracle.f32_to_f16_bits(up).astype(np.int64), nb | sb)
        assert np.array_equal(oracle.f32_to_f16_bits(dn).astype(np.int64), pos | sb)


def test_f16_rounding_matches_exact_definition_random():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 5, 3000),
                        rng.uniform(65000, 66000, 200)]).astype(np.float32)
    got = oracle.f32_to_f16_bits(v)
    ref = np.array([to_f16_bits(Fraction(float(t))) for t in v], np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("case", f16_cases()["quant"])
def test_f16_quant_hand_cases(case):
    xs, s, qs = case
    q, scale = oracle.quant_act(_bits(xs)[None, :], "f16")
    assert scale[0] == np.float32(s)
    assert q[0].tolist() == qs


@pytest.mark.parametrize("case", f16_cases()["epi"])
def test_f16_epilogue_hand_cases(case):
    acc, sa, sw, bias, y = case
    b = None if bias is None else np.array([bias], np.uint16)
    got = oracle.epilogue(np.array([[acc]], np.int32), np.array([sa], np.float32),
                          np.array([sw], np.float32), b, "f16")
    assert int(got[0, 0]) == y, hex(int(got[0, 0]))


def test_f16_epilogue_exact_rational_random():
    rng = np.random.default_rng(4)
    acc = rng.integers(-2**26, 2**26, size=(6, 7)).astype(np.int32)
    sa = (rng.uniform(0.5, 2, 6) * 10.0 ** rng.uniform(-6, -1, 6)).astype(np.float32)
    sw = (rng.uniform(0.5, 2, 7) * 10.0 ** rng.uniform(-5, -2, 7)).astype(np.float32)
    bias = oracle.f32_to_f16_bits(rng.standard_normal(7).astype(np.float32))
    got = oracle.epilogue(acc, sa, sw, bias, "f16")
    for m in range(6):
        for n in range(7):
            t = Fraction(float(np.float32(acc[m, n])))
            t = f32_mul(float(t), float(sa[m]))
            t = f32_mul(float(t), float(sw[n]))
            t = f32_add(float(t), float(_f16_value(int(bias[n]))))
            assert int(got[m, n]) == to_f16_bits(t), (m, n)


def test_f16_quant_exact_rational_random():
    rng = np.random.default_rng(5)
    rows = [rng.standard_normal(29) * 10.0 ** rng.uniform(-6, 4) for _ in range(16)]
    x = np.stack([oracle.f32_to_f16_bits(np.clip(r, -65504, 65504).astype(np.float32)) for r in rows])
    q, s = oracle.quant_act(x, "f16")
    xf = oracle.f16_bits_to_f32(x)
    for i in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in xf[i])
        es = f32_div(float(amax), 127.0)
        assert Fraction(float(s[i])) == es, i
        eq = [max(-127, min(127, round_half_even(f32_div(float(v), float(es))))) for v in xf[i]]
        assert q[i].tolist() == eq, i


@pytest.mark.parametrize("amax_bits", [0x3C00, 0x7BFF, 0x5BF0, 0x0001, 0x03FF, 0x0400, 0x4A3D])
def test_f16_quant_exhaustive(amax_bits):
    """All finite fp16 values below one amax, against the float64 route
    (fl32(fl64(a/b)) is the correctly rounded fp32 quotient)."""
    allv = oracle.f16_bits_to_f32(FINITE)
    amax = float(oracle.f16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
    vals = allv[np.abs(allv) <= amax]
    row = np.concatenate([[amax], vals]).astype(np.float32)
    x = oracle.f32_to_f16_bits(row)
    q, s = oracle.quant_act(x[None, :], "f16")
    s64 = np.float32(np.float64(amax) / 127.0)
    assert s[0] == s64
    ref = np.clip(np.rint((row.astype(np.float64) / np.float64(s64)).astype(np.float32)), -127, 127)
    assert np.array_equal(q[0].astype(np.float64), ref)


def test_f16_and_bf16_paths_agree_on_common_values():
    """Values held exactly by both formats quantise identically, and the
    epilogue gives the same fp32 value before the output cast."""
    rng = np.random.default_rng(6)
    xb = to_bf16_bits(rng.standard_normal((5, 64)))
    xv = oracle.bf16_bits_to_f32(xb)
    xh = _bits(xv)
    qb, sb = oracle.quant_act(xb)
    qh, sh = oracle.quant_act(xh, "f16")
    assert np.array_equal(qb, qh) and np.array_equal(sb, sh)
    wq = rng.integers(-127, 128, (9, 64)).astype(np.int8)
    sw = rng.uniform(1e-3, 1e-2, 9).astype(np.float32)
    bias_b = to_bf16_bits(rng.standard_normal(9) * 0.01)
    bias_h = _bits(oracle.bf16_bits_to_f32(bias_b))
    acc = oracle.gemm_exact(qb, wq)
    assert np.array_equal(oracle.epilogue_f32(acc, sb, sw, bias_b),
                          oracle.epilogue_f32(acc, sh, sw, bias_h, "f16"))


def test_f16_linear_against_dequantised_reference():
    """y is the fp16 rounding of the layer on its quantised operands: within
    half an fp16 ulp plus the fp32 steps of the float64 reference."""
    rng = np.random.default_rng(7)
    x = oracle.f32_to_f16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    w = oracle.f32_to_f16_bits((rng.standard_normal((24, 256)) * 0.02).astype(np.float32))
    bias = oracle.f32_to_f16_bits((rng.standard_normal(24) * 0.01).astype(np.float32))
    wq, sw = oracle.quantize_weights(w, "f16")
    r = oracle.linear(x, wq, sw, bias, "f16")
    ref = oracle.dequant_reference(r["xq"], r["s_a"], wq, sw) + \
        oracle.f16_bits_to_f32(bias).astype(np.float64)[None, :]
    y = oracle.f16_bits_to_f32(r["y"]).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0**-14))) - 10)
    assert np.all(np.abs(y - ref) <= 0.5 * ulp + 4 * 2.0**-24 * np.abs(ref) + 2.0**-25)
    assert oracle.rel_l2(y, ref) < 2.0**-11
