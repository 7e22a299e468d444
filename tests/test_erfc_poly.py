"""The GELU kernel's erfc polynomial (csrc/erfc_poly.h, written by
csrc/gen_erfc_poly.py): parsed from the header and checked against scipy's
erfc, CPU only. erfc(x) = t exp(-x^2 + P(t)), t = 1 / (1 + x/2), must stay
within 2 fp32 ulps over x in [0, 10] (every x where a bf16 GELU is not zero)
and decay to zero beyond."""
import os
import re

import numpy as np
from scipy.special import erfc

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "w8a8_int8_dynamic_quant_amd", "csrc", "erfc_poly.h")


def coefficients():
    text = open(HDR).read()
    body = text[text.index("kErfcPoly[kErfcPolyDegree + 1] = {"):]
    body = body[:body.index("};")]
    c = [float.fromhex(m) for m in re.findall(r"(-?0x[0-9a-fA-F.]+p[-+]?\d+)f", body)]
    deg = int(re.search(r"kErfcPolyDegree = (\d+);", text).group(1))
    assert len(c) == deg + 1
    assert all(np.float32(v) == v for v in c), "coefficients are fp32 values"
    return np.array(c)


def approx(x, c):
    t = 1 / (1 + 0.5 * x)
    return t * np.exp(-x * x + np.polyval(c[::-1], t))


def test_erfc_within_two_ulps():
    c = coefficients()
    x = np.linspace(0.0, 10.0, 1_000_001)
    rel = np.abs(approx(x, c) / erfc(x) - 1)
    assert rel.max() < 2 * 2.0**-24, rel.max()


def test_erfc_tail_and_origin():
    c = coefficients()
    assert abs(approx(np.array([0.0]), c)[0] - 1.0) < 2 * 2.0**-24
    x = np.array([10.0, 20.0, 1e3, 1e10])
    assert (approx(x, c) <= 1e-40).all()
    # P(0) is the limit -log(2 sqrt(pi)) of log(erfcx(x) / t) as x grows
    assert abs(c[0] + np.log(2 * np.sqrt(np.pi))) < 1e-6
