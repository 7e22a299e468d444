"""Pins of the oracle's fused producers (modulated LayerNorm and GELU, each
followed by the per-row int8 quantisation), CPU only.

What pins them, none of it calling the oracle's formulas back:
* hand-computed rows and the standard normal distribution table
  (tests/golden/producer_hand_cases.txt);
* libraries that implement the same functions independently: torch's float64
  layer_norm and gelu, the C library's erfc;
* identities of the definitions (GELU(z) - GELU(-z) = z; LayerNorm ignores a
  common offset and, with eps = 0, a common factor; its output has mean 0 and
  variance 1);
* the single bf16 rounding against exact rational rounding, including the
  values where rounding through fp32 first goes wrong;
* the fp32 error bounds against independent fp32 evaluations, and against
  being vacuous.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_arith import to_bf16_bits
from golden_io import producer_cases
from synth_inputs import all_finite_bf16, random_bf16, to_bf16_bits as to_bf16


def _bits(vals):
    return to_bf16(np.asarray(vals, np.float64))


# --- single rounding float64 -> bf16 -------------------------------------

def _rounding_cases():
    rng = np.random.default_rng(5)
    v = [0.0, -0.0, 1.0, 1 + 2**-8, 1 + 2**-8 + 2**-30, 1 + 2**-8 - 2**-40,
         1 + 3 * 2**-8, -(1 + 3 * 2**-8 + 2**-35), 2.0**-126, 2.0**-133, 2.0**-134,
         2.0**-134 + 2.0**-160, 3 * 2.0**-135, 2.0**-150, (2 - 2**-8) * 2.0**127,
         (2 - 2**-8) * 2.0**127 * (1 - 2**-40), 3e38, -1e39]
    # random values over the whole exponent range, and values within a few
    # fp64 ulps of bf16 midpoints (where a first rounding to fp32 lands on
    # the midpoint)
    v += list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 127, 300)))
    mids = (rng.integers(128, 256, 200) * 2 + 1).astype(np.float64) * np.exp2(
        rng.integers(-130, 110, 200).astype(np.float64))
    v += list(mids * (1 + rng.integers(-3, 4, 200) * 2.0**-52))
    v += list(mids * (1 + rng.choice([-1, 1], 200) * 2.0**-30))
    return np.array(v, np.float64)


def test_f64_to_bf16_single_rounding():
    v = _rounding_cases()
    got = oracle.f64_to_bf16_bits(v)
    for vi, gi in zip(v, got):
        exp = to_bf16_bits(Fraction(float(vi))) if vi != 0 else (0x8000 if math.copysign(1, vi) < 0 else 0)
        assert int(gi) == exp, (vi, hex(int(gi)), hex(exp))


def test_f64_to_bf16_double_rounding_trap():
    # 1 + 2^-8 + 2^-30 is nearer to 1 + 2^-7; through fp32 (RNE) it becomes the
    # midpoint 1 + 2^-8 and then rounds to even, 1.0
    assert int(oracle.f64_to_bf16_bits(np.array([1 + 2**-8 + 2**-30]))[0]) == 0x3F81
    assert int(oracle.f32_to_bf16_bits(np.array([1 + 2**-8 + 2**-30], np.float32))[0]) == 0x3F80


def test_bf16_within():
    f = oracle.bf16_within
    assert f(np.array([0x3F80, 0x3F81]), np.array([1 + 2**-8] * 2), 0.0).all()   # a tie: both
    assert not f(np.array([0x3F81]), np.array([1.0]), 0.0)[0]
    assert f(np.array([0x3F81]), np.array([1 + 2**-8 - 2**-20]), 2**-19)[0]
    assert not f(np.array([0x3F81]), np.array([1 + 2**-8 - 2**-20]), 2**-21)[0]
    assert f(np.array([0x3F80]), np.array([1 - 2**-30]), 0.0)[0]
    assert not f(np.array([0x3F7F]), np.array([1 - 2**-30]), 0.0)[0]
    assert f(np.array([0x7F80]), np.array([1e39]), 0.0)[0]
    assert not f(np.array([0x7F80]), np.array([1e38]), 0.0)[0]
    v = _rounding_cases()
    v = v[np.abs(v) < 3e38]
    assert f(oracle.f64_to_bf16_bits(v), v, 0.0).all()


# --- modulated LayerNorm --------------------------------------------------

def test_layernorm_hand_cases():
    ln, _ = producer_cases()
    assert len(ln) >= 4
    for x, sh, sc, eps, v, q in ln:
        got = oracle.layernorm_modulate(_bits([x]), _bits([sh]), _bits([sc]), eps)
        np.testing.assert_allclose(got[0], v, rtol=1e-14, atol=1e-15)
        if q is not None:
            r = oracle.layernorm_modulate_quant(_bits([x]), _bits([sh]), _bits([sc]), eps)
            assert r["xq"][0].tolist() == q
            assert np.array_equal(r["y"][0], _bits(v))


@pytest.mark.parametrize("seed", range(4))
def test_layernorm_against_torch(seed):
    rng = np.random.default_rng(seed)
    M, K, rpg = 10, 96, 4
    G = (M + rpg - 1) // rpg
    x = random_bf16(rng, (M, K), [1.0, 30.0, 1e-3, 3.0][seed])
    sh, sc = random_bf16(rng, (G, K), 0.5), random_bf16(rng, (G, K), 0.3)
    eps = [1e-6, 1e-5, 1e-2, 1e-6][seed]
    got = oracle.layernorm_modulate(x, sh, sc, eps, rows_per_group=rpg)
    xt = torch.from_numpy(oracle.bf16_bits_to_f32(x).astype(np.float64))
    for g in range(G):
        rows = slice(g * rpg, min(M, (g + 1) * rpg))
        w = torch.from_numpy(1.0 + oracle.bf16_bits_to_f32(sc[g]).astype(np.float64))
        b = torch.from_numpy(oracle.bf16_bits_to_f32(sh[g]).astype(np.float64))
        ref = torch.nn.functional.layer_norm(xt[rows], (K,), w, b, float(np.float32(eps)))
        np.testing.assert_allclose(got[rows], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_layernorm_invariants():
    rng = np.random.default_rng(11)
    M, K = 6, 64
    # small integers: x + 16 and 4 x are exact in bf16
    xi = rng.integers(-40, 41, (M, K)).astype(np.float64)
    zero = np.zeros((1, K), np.uint16)
    base = oracle.layernorm_modulate(_bits(xi), zero, zero, 0.0)
    assert np.abs(base.mean(axis=1)).max() < 1e-14
    np.testing.assert_allclose((base * base).mean(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.layernorm_modulate(_bits(xi + 16), zero, zero, 0.0), base,
                               rtol=1e-12, atol=1e-13)
    assert np.array_equal(oracle.layernorm_modulate(_bits(4 * xi), zero, zero, 0.0), base)
    # rows use the shift/scale of their group
    sh, sc = random_bf16(rng, (3, K), 1.0), random_bf16(rng, (3, K), 1.0)
    grouped = oracle.layernorm_modulate(_bits(xi), sh, sc, 1e-6, rows_per_group=2)
    for m in range(M):
        one = oracle.layernorm_modulate(_bits(xi[m:m + 1]), sh[m // 2], sc[m // 2], 1e-6)
        assert np.array_equal(grouped[m], one[0])


# --- GELU -----------------------------------------------------------------

def test_gelu_standard_normal_table():
    _, ge = producer_cases()
    assert len(ge) >= 6
    for z, phi in ge:
        got = oracle.gelu(_bits([z]))[0]
        assert got == pytest.approx(z * phi, rel=1e-12, abs=1e-300), (z, got, z * phi)
        assert oracle.gelu(_bits([z]), "tanh")[0] == pytest.approx(z * phi, abs=1e-3)
    assert oracle.gelu(_bits([0.0]), "tanh")[0] == 0.0


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_odd_part_identity(approximate):
    """GELU(z) - GELU(-z) = z for both forms, over every finite bf16 z."""
    z = all_finite_bf16()
    pos = oracle.gelu(z, approximate)
    neg = oracle.gelu(z ^ np.uint16(0x8000), approximate)
    zf = oracle.bf16_bits_to_f32(z).astype(np.float64)
    np.testing.assert_allclose(pos - neg, zf, rtol=4e-16, atol=0)


def test_gelu_erf_against_libm():
    z = all_finite_bf16()
    zf = oracle.bf16_bits_to_f32(z).astype(np.float64)
    ref = np.array([0.5 * t * math.erfc(-t / math.sqrt(2.0)) for t in zf])
    np.testing.assert_allclose(oracle.gelu(z), ref, rtol=1e-13, atol=1e-300)  # fp64 subnormals


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_against_torch(approximate):
    """torch's float64 gelu, where its 1 + erf / 1 + tanh does not cancel (z >= -5)."""
    z = all_finite_bf16()
    zf = oracle.bf16_bits_to_f32(z).astype(np.float64)
    keep = (zf >= -5.0) & (zf <= 1e30)
    ref = torch.nn.functional.gelu(torch.from_numpy(zf[keep]), approximate=approximate).numpy()
    np.testing.assert_allclose(oracle.gelu(z[keep], approximate), ref, rtol=1e-9, atol=1e-300)


def test_gelu_tanh_close_to_erf():
    z = all_finite_bf16()
    zf = oracle.bf16_bits_to_f32(z).astype(np.float64)
    keep = np.abs(zf) <= 10.0
    d = np.abs(oracle.gelu(z[keep], "tanh") - oracle.gelu(z[keep]))
    assert d.max() < 1e-3 and d.max() > 1e-5


# --- the fp32 error bounds --------------------------------------------------

def _ln_fp32_sequential(x_bits, sh_bits, sc_bits, eps):
    """An fp32 evaluation with sequential (left to right) sums."""
    x = oracle.bf16_bits_to_f32(x_bits)
    K = x.shape[1]
    s = np.add.accumulate(x, axis=1, dtype=np.float32)[:, -1:]
    mean = s / np.float32(K)
    d = x - mean
    var = np.add.accumulate(d * d, axis=1, dtype=np.float32)[:, -1:] / np.float32(K)
    rstd = np.float32(1) / np.sqrt(var + np.float32(eps))
    g = np.float32(1) + oracle.bf16_bits_to_f32(sc_bits)
    return ((d * rstd) * g + oracle.bf16_bits_to_f32(sh_bits)).astype(np.float64)


def _ln_fp32_blocked(x_bits, sh_bits, sc_bits, eps, lanes=64):
    """An fp32 evaluation whose row sums run sequentially in `lanes` strided
    runs, then add the runs pairwise: depth K/lanes - 1 + log2(lanes)."""
    x = oracle.bf16_bits_to_f32(x_bits)
    M, K = x.shape

    def rowsum(a):
        part = np.add.accumulate(a.reshape(M, K // lanes, lanes), axis=1, dtype=np.float32)[:, -1]
        while part.shape[1] > 1:
            part = part[:, 0::2] + part[:, 1::2]
        return part

    mean = rowsum(x) / np.float32(K)
    d = x - mean
    var = rowsum(d * d) / np.float32(K)
    rstd = np.float32(1) / np.sqrt(var + np.float32(eps))
    g = np.float32(1) + oracle.bf16_bits_to_f32(sc_bits)
    return ((d * rstd) * g + oracle.bf16_bits_to_f32(sh_bits)).astype(np.float64)


def _ln_case(seed, K=3072, M=8, offset=0.0):
    rng = np.random.default_rng(100 + seed)
    x = to_bf16(oracle.bf16_bits_to_f32(random_bf16(rng, (M, K), 1.0)) + offset)
    x[:, rng.choice(K, 15, replace=False)] = random_bf16(rng, (M, 15), 30.0)
    return x, random_bf16(rng, (1, K), 0.5), random_bf16(rng, (1, K), 0.5)


@pytest.mark.parametrize("seed", range(3))
def test_layernorm_bound_any_order(seed):
    x, sh, sc = _ln_case(seed, offset=[0.0, 3.0, -20.0][seed])
    v = oracle.layernorm_modulate(x, sh, sc, 1e-6)
    v32 = _ln_fp32_sequential(x, sh, sc, 1e-6)
    assert (np.abs(v32 - v) <= oracle.layernorm_modulate_err_bound(x, sh, sc, 1e-6)).all()


@pytest.mark.parametrize("seed", range(3))
def test_layernorm_bound_blocked_holds_and_is_tight(seed):
    x, sh, sc = _ln_case(seed, offset=[0.0, 3.0, -20.0][seed])
    K = x.shape[1]
    v = oracle.layernorm_modulate(x, sh, sc, 1e-6)
    bound = oracle.layernorm_modulate_err_bound(x, sh, sc, 1e-6, depth=K // 64 + 16)
    v32 = _ln_fp32_blocked(x, sh, sc, 1e-6)
    assert (np.abs(v32 - v) <= bound).all()
    # sharp: a parity test accepts the other bf16 neighbour of v only within
    # `bound` of a midpoint, on about 2 bound / ulp of the elements (a row
    # offset far from zero makes the fp32 mean, and so the bound, coarser)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 2.0**-126))[1] - 8)
    assert np.mean(bound / ulp) < [0.02, 0.05, 0.3][seed]


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_bound_holds_and_is_tight(approximate):
    z = all_finite_bf16()
    zf = oracle.bf16_bits_to_f32(z)
    keep = np.abs(zf) < 1e18          # z^3 stays finite in fp32
    z, zf = z[keep], torch.from_numpy(zf[keep])
    if approximate == "none":
        v32 = (0.5 * zf * torch.special.erfc(-zf * np.float32(1 / math.sqrt(2)))).double().numpy()
    else:
        t = np.float32(math.sqrt(2 / math.pi)) * (zf + np.float32(0.044715) * (zf * zf * zf))
        e = torch.exp(-2 * t.abs())
        v32 = torch.where(t >= 0, zf / (1 + e), zf * e / (1 + e)).double().numpy()
    v = oracle.gelu(z, approximate)
    bound = oracle.gelu_err_bound(z, approximate)
    assert (np.abs(v32 - v) <= bound).all()
    small = np.abs(zf.numpy()) < 8
    half_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 2.0**-126))[1] - 9)
    assert np.mean((bound < half_ulp / 8)[small]) > 0.99
