"""The GELU producer's build-time tables (csrc/gen_gelu_table.cpp: GELU in
double precision, rounded once to the nearest bf16), CPU only.

The generator is the product's own host program: build_lib runs it at build
time, and the library's GELU kernel looks its output up on the GPU (the GPU
tests compare the kernel's output with these tables on every finite bf16
input). Here it is built and run on the host, and each of its 65536-entry
tables is checked against the oracle: for every finite bf16 z the entry must
be a correct bf16 result for the exact GELU(z) within the bound the oracle
derives (oracle.gelu_err_bound), and it must be the nearest bf16 to the
oracle's float64 GELU(z) (two entries of slack for a value within a few
float64 ulps of a bf16 midpoint, where two float64 evaluations may round
apart)."""
import re
import shutil

import numpy as np
import pytest

import oracle
from synth_inputs import all_finite_bf16

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


@pytest.fixture(scope="module")
def tables(tmp_path_factory):
    from w8a8_int8_dynamic_quant_amd import build_lib
    out = build_lib.gen_gelu_table(build_dir=str(tmp_path_factory.mktemp("gelu")))
    text = open(out).read()
    vals = [int(v, 16) for v in re.findall(r"0x([0-9a-f]{4}),", text)]
    assert len(vals) == 2 * 65536
    return np.array(vals, np.uint16).reshape(2, 65536)


@pytest.mark.parametrize("form,approximate", [(0, "none"), (1, "tanh")])
def test_every_finite_bf16_within_bound(tables, form, approximate):
    z = all_finite_bf16()
    y = tables[form][z]
    v = oracle.gelu(z, approximate)
    ok = oracle.bf16_within(y, v, oracle.gelu_err_bound(z, approximate))
    assert ok.all(), (z[~ok][:5], y[~ok][:5], v[~ok][:5])
    not_nearest = int(np.count_nonzero(y != oracle.f64_to_bf16_bits(v)))
    assert not_nearest <= 2, not_nearest


def test_zero_infinities_and_signs(tables):
    # GELU(+-0) = +-0 and GELU(+inf) = +inf, GELU(-inf) = -0 (the limits) in
    # both forms; GELU(z) > 0 for z > 0, <= 0 for z < 0
    for form in (0, 1):
        assert tables[form][0x7F80] == 0x7F80 and tables[form][0xFF80] == 0x8000
    z = all_finite_bf16()
    neg = (z & 0x8000) != 0
    for form in (0, 1):
        t = tables[form]
        assert t[0x0000] == 0x0000 and t[0x8000] == 0x8000
        y = t[z]
        nonzero = (y & 0x7FFF) != 0
        assert np.all(((y & 0x8000) != 0)[nonzero] == neg[nonzero])


def test_deterministic(tables, tmp_path):
    from w8a8_int8_dynamic_quant_amd import build_lib
    out = build_lib.gen_gelu_table(build_dir=str(tmp_path))
    vals = np.array([int(v, 16) for v in re.findall(r"0x([0-9a-f]{4}),", open(out).read())], np.uint16)
    assert np.array_equal(vals.reshape(2, 65536), tables)
