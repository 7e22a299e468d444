"""Whole-layer pins of the oracle against the pages' accuracy figures.

The Issue 5 probe ("Round two" section) reports that the int8 ops match a
float32 reference at 0.17% rel-L2 on (64,256,128), (512,4096,4096) and
(512,4096,12288), and that leaving act_scale out of the reference makes the
out/ref norm ratio equal E[act_scale] (the 97% error scare). These tests pin
the oracle to those observations and to a noise model of the unquantised
product.
"""
import numpy as np
import pytest

import oracle
from synth_inputs import SPECS, LinearSpec, make_linear_inputs


def _run(name):
    d = make_linear_inputs(name)
    wq, s_w = oracle.quantize_weights(d["w"])
    out = oracle.linear(d["x"], wq, s_w, d["bias"])
    return d, wq, s_w, out


CASES = ["c1_64x256x128", "c2_512x4096x4096_outliers", "c3_512x4096x12288_student_t"]


@pytest.mark.parametrize("name", CASES)
def test_layer_matches_dequantized_reference_at_017pct(name):
    """Against (xq*s_a)(wq*s_w)^T (+bias), only the bf16 output rounding is
    left: rel-L2 about 0.17% as the pages report (bf16 rounding of a smooth
    distribution gives 2^-8/sqrt(12)*sqrt(E[x^2]/..) ~ 0.166%)."""
    d, wq, s_w, out = _run(name)
    ref = oracle.dequant_reference(out["xq"], out["s_a"], wq, s_w, d["bias"])
    y = oracle.bf16_bits_to_f32(out["y"])
    r = oracle.rel_l2(y, ref)
    assert 0.0015 < r < 0.0018, r
    # every element is within half a bf16 ulp of the float64 value, plus the
    # fp32 epilogue's own rounding of its terms (a few 2^-24 of |product| and
    # |bias|, which matters where the bias cancels the product) and float64
    # cancellation noise where the exact integer sum is zero
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2**16
    b = 0.0 if d["bias"] is None else oracle.bf16_bits_to_f32(d["bias"]).astype(np.float64)
    terms = np.abs(ref - b) + np.abs(b)
    tol = 0.5 * ulp + 2.0**-21 * terms + 1e-12 * np.abs(ref).max()
    assert np.all(np.abs(y - ref) <= tol)


@pytest.mark.parametrize("name", CASES)
def test_layer_against_unquantised_matches_noise_model(name):
    d, wq, s_w, out = _run(name)
    ref = oracle.float_reference(d["x"], d["w"], d["bias"])
    y = oracle.bf16_bits_to_f32(out["y"])
    measured = oracle.rel_l2(y, ref)
    model = oracle.noise_model_rel_l2(d["x"], d["w"], out["xq"], out["s_a"], wq, s_w)
    assert abs(measured / model - 1.0) < 0.05, (measured, model)
    # quantisation noise is well above bf16 rounding and well below 100%
    assert 0.005 < measured < 0.2


def test_negative_control_missing_act_scale():
    """Dropping s_a from the reference makes out/ref ~= E[s_a]."""
    # the pages' case: plain Gaussian activations of width 4096
    spec = LinearSpec("gauss", 512, 4096, 4096)
    d = make_linear_inputs(spec)
    wq, s_w = oracle.quantize_weights(d["w"])
    out = oracle.linear(d["x"], wq, s_w, None)
    bad_ref = oracle.dequant_reference(out["xq"], np.ones_like(out["s_a"]), wq, s_w)
    y = oracle.bf16_bits_to_f32(out["y"])
    ratio = np.linalg.norm(y) / np.linalg.norm(bad_ref)
    e_s = float(np.mean(out["s_a"]))
    assert abs(ratio / e_s - 1.0) < 0.02
    assert 0.025 < e_s < 0.035                 # ~ E[max|N(0,1)| over 4096] / 127
    assert oracle.rel_l2(y, bad_ref) > 0.95


def test_layer_intermediates_consistent():
    d, wq, s_w, out = _run("c1_64x256x128")
    assert out["xq"].dtype == np.int8 and out["s_a"].dtype == np.float32
    assert out["acc"].dtype == np.int32 and out["y"].dtype == np.uint16
    exp = oracle.gemm_int64_rows(out["xq"], wq)
    assert np.array_equal(out["acc"].astype(np.int64), exp)


def test_inputs_are_deterministic_and_shaped():
    a = make_linear_inputs("c1_64x256x128")
    b = make_linear_inputs("c1_64x256x128")
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["x"].shape == (64, 256) and a["w"].shape == (128, 256)
    assert a["bias"].shape == (128,)
    for name, s in SPECS.items():
        assert s.K % 16 == 0, name
