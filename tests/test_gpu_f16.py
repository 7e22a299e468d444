"""GPU parity of the fp16 entry points (w8a8_*_f16, through the C ABI)
against the oracle's fp16 variant.

Same bar as the bf16 layer: xq, a_scale, wq, w_scale and the int32
accumulators bit-exact; fp16 outputs within 1 fp16 ulp (the epilogue follows
the oracle's fp32 order, so they are expected bit-identical; the count of
differing elements is reported). Infinities from fp16 overflow compare as
values (the ulp distance of +-inf to itself is 0)."""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, assert_bf16_close, assert_equal, dev, dev_f16, host, host_bits
from synth_inputs import all_finite_f16, random_f16, to_f16_bits

pytestmark = pytest.mark.gpu

F16 = "f16"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _check_quant(x_bits, fn="act", ld=None):
    R, K = x_bits.shape
    if ld is not None and ld != K:
        pad = np.zeros((R, ld), np.uint16)
        pad[:, :K] = x_bits
        xd = dev_f16(pad)[:, :K]
    else:
        xd = dev_f16(x_bits)
    q, s = (w8.quant_act if fn == "act" else w8.quantize_weights)(xd)
    torch.cuda.synchronize()
    eq, es = oracle.quant_act(x_bits, F16)
    assert_equal(host(s), es, "scale")
    assert_equal(host(q), eq, "q")


def test_f16_quant_exhaustive_sweep():
    """Rows enumerate every finite fp16 value below several amax values
    (1, 65504, a non-power-of-two, the smallest subnormal, the largest
    subnormal, the smallest normal); the widest row takes the two-pass
    kernel."""
    allv = all_finite_f16()
    vals = oracle.f16_bits_to_f32(allv)
    rows = []
    for amax_bits in (0x3C00, 0x7BFF, 0x5BF0, 0x0001, 0x03FF, 0x0400, 0x4A3D):
        amax = oracle.f16_bits_to_f32(np.array([amax_bits], np.uint16))[0]
        sel = allv[np.abs(vals) <= amax]
        rows.append(np.concatenate([[amax_bits], sel]))
    K = (max(len(r) for r in rows) + 15) // 16 * 16
    x = np.zeros((len(rows), K), np.uint16)
    for i, r in enumerate(rows):
        x[i, : len(r)] = r
    announce(f"f16 quant exhaustive sweep {x.shape}")
    _check_quant(x, "act")


@pytest.mark.parametrize("R,K,ld", [(1, 16, 16), (3, 48, 64), (5, 1040, 1040), (7, 3072, 3080),
                                    (3, 2064, 2072), (5, 3088, 3096), (3, 14000, 14000),
                                    (2049, 4112, 4120),
                                    (9, 4096, 4096), (4, 12288, 12288), (3, 16400, 16408),
                                    (2, 40000, 40000), (3, 4112, 4120), (2, 8192, 8192),
                                    (2, 24592, 24600), (3, 32768, 32768)])
def test_f16_quant_ragged_and_strided(R, K, ld):
    rng = np.random.default_rng(R * 7 + K)
    x = random_f16(rng, (R, K), 10.0)
    announce(f"f16 quant R={R} K={K} ld={ld}")
    _check_quant(x, "act", ld)
    _check_quant(x, "w", ld)


def _linear_case(x_bits, w_bits, bias_bits, ldx=None, ldo=None):
    """w8a8_linear_f16 and w8a8_scaled_mm_f16 against the oracle."""
    M, K = x_bits.shape
    N = w_bits.shape[0]
    wq_e, sw_e = oracle.quantize_weights(w_bits, F16)
    exp = oracle.linear(x_bits, wq_e, sw_e, bias_bits, F16)
    wq, sw = w8.quantize_weights(dev_f16(w_bits))
    if ldx is not None and ldx != K:
        # the padding holds 32768.0: read into any row's amax, it would
        # change that row's scale and every code
        xpad = np.full((M, ldx), 0x7800, np.uint16)
        xpad[:, :K] = x_bits
        xd = dev_f16(xpad)[:, :K]
    else:
        xd = dev_f16(x_bits)
    bd = None if bias_bits is None else dev_f16(bias_bits)
    out_full = None
    if ldo is not None and ldo != N:
        # a sentinel in the output's padding columns, checked after the call
        out_full = dev_f16(np.full((M, ldo), 0x1234, np.uint16))
        out = out_full[:, :N]
    else:
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(w8.workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device="cuda")
    w8.linear(xd, wq, sw, bd, out=out, workspace=ws, acc_debug=acc)
    torch.cuda.synchronize()
    assert_equal(host(sw), sw_e, "w_scale")
    assert_equal(host(wq), wq_e, "wq")
    xq_d, sa_d = w8.workspace_views(ws, M, K)
    assert_equal(host(sa_d), exp["s_a"], "a_scale")
    assert_equal(host(xq_d), exp["xq"], "xq")
    assert_equal(host(acc), exp["acc"], "acc")
    stats = assert_bf16_close(host_bits(out), exp["y"])
    if out_full is not None:
        assert (host_bits(out_full)[:, N:] == 0x1234).all(), "output padding written"
    out2 = w8.scaled_mm(dev(exp["xq"]), dev(exp["s_a"]), wq, sw, bd, dtype=torch.float16)
    torch.cuda.synchronize()
    assert out2.dtype == torch.float16
    assert_bf16_close(host_bits(out2), exp["y"])
    return stats, exp


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 48), (16, 70, 8192), (2, 129, 8208),
                                   (40, 72, 4112), (20, 40, 8192), (3, 40, 24592), (2, 24, 32768),
                                   (17, 33, 64), (25, 70, 1040), (32, 200, 3072), (13, 18432, 1024),
                                   (20, 18432, 1024), (32, 18432, 1024), (65, 129, 1040),
                                   (257, 513, 256), (300, 700, 1296)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_f16_linear_shapes(M, N, K, with_bias):
    rng = np.random.default_rng(M * 1000 + N + K + 5)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01) if with_bias else None
    announce(f"f16 linear M={M} N={N} K={K} bias={with_bias} path={w8.linear_path(M, K, N)}")
    print(_linear_case(x, w, b)[0])


@pytest.mark.parametrize("M,N,K", [(4352, 9216, 3072), (1, 18432, 3072), (16, 18432, 3072)])
def test_f16_linear_full_size(M, N, K):
    rng = np.random.default_rng(M + N)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01) if M <= 16 else None
    announce(f"f16 linear full size M={M} N={N} K={K}")
    print(_linear_case(x, w, b)[0])


@pytest.mark.parametrize("M,K,ldx", [(5, 256, 264), (40, 256, 264), (12, 256, 264), (3, 3088, 3096)])
def test_f16_linear_strided_x_and_out(M, K, ldx):
    """As the bf16 strided test: small-M row modes, the split kernel's staged
    and two-pass rows, the GEMM path."""
    rng = np.random.default_rng(22 + M)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (72, K), 0.02)
    announce(f"f16 linear strided M={M} K={K} ldx={ldx}")
    _linear_case(x, w, None, ldx=ldx, ldo=75)


def test_f16_overflow_and_subnormal_outputs():
    """Outputs past 65504 become +-inf and tiny ones fp16 subnormals, on
    both the small-M kernel and the GEMM."""
    rng = np.random.default_rng(23)
    K, N = 256, 96
    for M in (6, 80):
        big = rng.choice([-1.0, 1.0], (M // 2, K)) * 1000.0
        tiny = rng.normal(0.0, 1.0, (M - M // 2, K)) * 6.5e-5
        x = to_f16_bits(np.concatenate([big, tiny]))
        w = to_f16_bits(np.concatenate([np.full((N // 2, K), 4.0),
                                        rng.normal(0.0, 1e-4, (N - N // 2, K))]))
        announce(f"f16 overflow/subnormal outputs M={M}")
        _, exp = _linear_case(x, w, None)
        y = oracle.f16_bits_to_f32(exp["y"])
        assert np.any(np.isinf(y))
        assert np.any((np.abs(y) > 0) & (np.abs(y) < 2.0**-14))


def test_f16_and_bf16_weights_interchangeable():
    """wq / w_scale from the fp16 quantiser serve the bf16 layer and give the
    same integer accumulators (values both formats hold)."""
    rng = np.random.default_rng(24)
    wb = to_f16_bits(np.round(rng.normal(0, 0.02, (40, 128)) * 2**12) / 2**12)
    xb = to_f16_bits(np.round(rng.normal(0, 1, (20, 128)) * 64) / 64)
    wq16, sw16 = w8.quantize_weights(dev_f16(wb))
    wq_e, sw_e = oracle.quantize_weights(wb, F16)
    acc = torch.empty((20, 40), dtype=torch.int32, device="cuda")
    xq, sa = w8.quant_act(dev_f16(xb))
    w8.scaled_mm(xq, sa, wq16, sw16, acc_debug=acc)           # bf16 output
    torch.cuda.synchronize()
    exp = oracle.linear(xb, wq_e, sw_e, None, F16)
    assert_equal(host(acc), exp["acc"], "acc")


@pytest.mark.parametrize("N", [2056, 2052, 2050])
def test_f16_256_tile_with_bias(N):
    """fp16 bias and output through the 256x256 tile's three store paths."""
    M, K = 4352, 272
    assert w8.gemm_tile(M, K, N) == (256, 256)
    rng = np.random.default_rng(N + 77)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01)
    announce(f"f16 256 tile M={M} N={N} K={K} bias")
    print(_linear_case(x, w, b)[0])


def test_f16_linear_split_k():
    """fp16 output and bias through the split-K reduction (see the bf16 test)."""
    M, N, K = 512, 4104, 2000
    assert w8.gemm_tile(M, K, N) == (128, 128)
    assert w8.workspace_bytes(M, K, N) > M * K + 4 * M + 512
    rng = np.random.default_rng(41)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01)
    announce(f"fp16 split-K linear M={M} N={N} K={K}")
    _linear_case(x, w, b)


def test_f16_linear_256_tile_halves():
    """fp16 output and bias with every 256x256 tile run as two 128-row halves
    (99 tiles, at most half of the compute units)."""
    M, N, K = 700, 8200, 2000
    assert w8.gemm_tile(M, K, N) == (256, 256)
    assert w8.workspace_bytes(M, K, N) < M * K + 4 * M + 512
    rng = np.random.default_rng(43)
    x = random_f16(rng, (M, K))
    w = random_f16(rng, (N, K), 0.02)
    b = random_f16(rng, (N,), 0.01)
    announce(f"fp16 256 tile halves M={M} N={N} K={K}")
    _linear_case(x, w, b)
