"""GPU parity of the W8A16 small-M linear (w8a16_linear: int8 weights, bf16
activations, fp32 accumulation) against the oracle.

The kernel accumulates in fp32 in the MFMA's order, the oracle takes the sum
in float64 and rounds it once, so the bar is a tolerance derived from the
arithmetic: with n fp32 accumulation steps per output (two MFMAs per
128-element window plus the final pair sum), |acc_gpu - acc| <= (2n + 8) *
2^-24 * sum_k |x[k] wq[n,k]|; that error scaled by |s_w| plus one bf16 ulp of
the result (a rounding boundary may fall in between) bounds |y_gpu - y|.
The count of outputs that differ at all is reported."""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, dev_bf16, dev_f16, host_bits
from synth_inputs import make_linear_inputs, random_bf16, random_f16, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _ulp(v, dtype="bf16"):
    """One ulp of the output type at |v| (bf16: 8 significant bits, smallest
    subnormal 2^-133; fp16: 11 bits, 2^-24)."""
    v = np.abs(np.asarray(v, np.float64))
    bits, tiny = (7, -133) if dtype == "bf16" else (10, -24)
    e = np.floor(np.log2(np.maximum(v, 2.0**tiny)))
    return np.maximum(2.0 ** (e - bits), 2.0**tiny)


def check_w8a16(x_bits, wq, sw, bias_bits, y_bits, dtype="bf16") -> dict:
    exp = oracle.w8a16_linear(x_bits, wq, sw, bias_bits, dtype)
    err = oracle.w8a16_err_bound(x_bits, wq, sw, dtype)
    y = oracle.to_f32(y_bits, dtype).astype(np.float64)
    ye = oracle.to_f32(exp["y"], dtype).astype(np.float64)
    assert np.all(np.isfinite(ye)), "the cases stay inside the output range"
    tol = err + _ulp(np.maximum(np.abs(y), np.abs(ye)), dtype)
    bad = np.abs(y - ye) > tol
    stats = {"n": int(y.size), "n_diff": int(np.count_nonzero(y_bits != exp["y"])),
             "max_excess": float(np.max(np.abs(y - ye) - tol)) if y.size else 0.0}
    assert not bad.any(), (stats, np.argwhere(bad)[:5])
    return stats


def _case(M, K, N, with_bias, ldx=None, ldo=None, seed=0):
    rng = np.random.default_rng(seed + M * 7 + K + N)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    wq_e, sw_e = oracle.quantize_weights(w)
    wq, sw = w8.quantize_weights(dev_bf16(w))
    if ldx is not None:
        xpad = np.zeros((M, ldx), np.uint16)
        xpad[:, :K] = x
        xd = dev_bf16(xpad)[:, :K]
    else:
        xd = dev_bf16(x)
    out = None
    if ldo is not None:
        out = torch.empty((M, ldo), dtype=torch.bfloat16, device="cuda")[:, :N]
    announce(f"w8a16 M={M} K={K} N={N} bias={with_bias} ldx={ldx} ldo={ldo}")
    y = w8.w8a16_linear(xd, wq, sw, None if b is None else dev_bf16(b), out=out)
    torch.cuda.synchronize()
    return check_w8a16(x, wq_e, sw_e, b, host_bits(y))


@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (3, 48, 70), (5, 1040, 129), (8, 3072, 100),
                                   (9, 512, 33), (16, 3968, 100), (2, 8064, 40), (8, 8064, 24)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a16_shapes(M, K, N, with_bias):
    print(_case(M, K, N, with_bias))


def test_w8a16_strided():
    print(_case(5, 256, 72, True, ldx=264, ldo=75))


@pytest.mark.parametrize("m", [1, 2, 8, 16])
def test_w8a16_modulation_full_size(m):
    d = make_linear_inputs(f"mod_m{m}_3072x18432")
    wq_e, sw_e = oracle.quantize_weights(d["w"])
    wq, sw = w8.quantize_weights(dev_bf16(d["w"]))
    announce(f"w8a16 modulation M={m}")
    y = w8.w8a16_linear(dev_bf16(d["x"]), wq, sw, dev_bf16(d["bias"]))
    torch.cuda.synchronize()
    print(m, check_w8a16(d["x"], wq_e, sw_e, d["bias"], host_bits(y)))


def test_w8a16_mixed_magnitudes():
    """Activations spread over many binades (cancellation in the sum) stay
    within the derived bound."""
    rng = np.random.default_rng(23)
    M, K, N = 4, 3072, 256
    mag = 2.0 ** rng.integers(-20, 10, (M, K))
    x = to_bf16_bits(rng.standard_normal((M, K)) * mag)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-3, 1e-1, N).astype(np.float32)
    announce("w8a16 mixed magnitudes")
    y = w8.w8a16_linear(dev_bf16(x), torch.from_numpy(wq).cuda(), torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    print(check_w8a16(x, wq, sw, None, host_bits(y)))


# ---- fp16 activations, bias and output (w8a16_linear_f16) -----------------

@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (3, 48, 70), (5, 1040, 129), (9, 512, 33),
                                   (16, 3968, 100), (8, 8064, 24)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a16_f16_shapes(M, K, N, with_bias):
    rng = np.random.default_rng(M * 11 + K + N)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01) if with_bias else None
    wq_e, sw_e = oracle.quantize_weights(w, "f16")
    wq, sw = w8.quantize_weights(dev_f16(w))
    announce(f"w8a16 f16 M={M} K={K} N={N} bias={with_bias}")
    y = w8.w8a16_linear(dev_f16(x), wq, sw, None if b is None else dev_f16(b))
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    print(check_w8a16(x, wq_e, sw_e, b, host_bits(y), "f16"))


@pytest.mark.parametrize("m", [1, 16])
def test_w8a16_f16_modulation_full_size(m):
    rng = np.random.default_rng(31 + m)
    x = random_f16(rng, (m, 3072))
    w = random_f16(rng, (18432, 3072), 0.02)
    b = random_f16(rng, (18432,), 0.01)
    wq_e, sw_e = oracle.quantize_weights(w, "f16")
    wq, sw = w8.quantize_weights(dev_f16(w))
    announce(f"w8a16 f16 modulation M={m}")
    y = w8.w8a16_linear(dev_f16(x), wq, sw, dev_f16(b))
    torch.cuda.synchronize()
    print(m, check_w8a16(x, wq_e, sw_e, b, host_bits(y), "f16"))


def test_w8a16_f16_every_weight_value():
    """Every int8 weight value -128..127 (the widening's whole domain, -128
    included as ingest may produce it) against one-hot activations: the
    outputs are the weights times the scale, exactly."""
    K, N = 256, 16
    wq = ((np.arange(N * K) % 256) - 128).astype(np.int8).reshape(N, K)
    x = np.zeros((8, K), np.float64)
    for t in range(8):
        x[t, 37 * t % K] = 1.0
    xb = to_f16_bits_exact(x)
    sw = np.full(N, 0.5, np.float32)
    announce("w8a16 f16 every weight value")
    y = w8.w8a16_linear(dev_f16(xb), torch.from_numpy(wq).cuda(), torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    got = oracle.f16_bits_to_f32(host_bits(y)).astype(np.float64)
    want = np.stack([wq[:, 37 * t % K].astype(np.float64) * 0.5 for t in range(8)])
    assert np.array_equal(got, want)


def to_f16_bits_exact(a):
    from synth_inputs import to_f16_bits
    b = to_f16_bits(a)
    assert np.array_equal(oracle.f16_bits_to_f32(b).astype(np.float64), a)
    return b
