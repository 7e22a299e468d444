"""GPU parity of libw8a8 (through its C ABI) against the CPU oracle.

Bar: xq, a_scale, wq, w_scale and the int32 accumulators bit-exact; bf16
outputs within 1 bf16 ulp (the epilogue is written in the oracle's fp32
order, so they are expected to be bit-identical and the count of differing
elements is reported).
"""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import (announce, assert_bf16_close, assert_equal, dev, dev_bf16, host,
                      host_bits)
from synth_inputs import (SPECS, LinearSpec, all_finite_bf16, make_linear_inputs,
                          random_bf16, to_bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- quantisation

def _check_quant(x_bits, fn="act"):
    xd = dev_bf16(x_bits)
    q, s = (w8.quant_act if fn == "act" else w8.quantize_weights)(xd)
    torch.cuda.synchronize()
    eq, es = oracle.quant_act(x_bits)
    assert_equal(host(s), es, "scale")
    assert_equal(host(q), eq, "q")


@pytest.mark.parametrize("name", ["c1_64x256x128", "c2_512x4096x4096_outliers",
                                  "c3_512x4096x12288_student_t", "dit_down_4352x12288x3072"])
def test_quant_act_configs(name):
    d = make_linear_inputs(name)
    announce(f"quant_act {name} {d['x'].shape}")
    _check_quant(d["x"], "act")


@pytest.mark.parametrize("name", ["c1_64x256x128", "dit_up_4352x3072x12288",
                                  "mod_m1_3072x18432"])
def test_quantize_weights_configs(name):
    d = make_linear_inputs(name)
    announce(f"quantize_weights {name} {d['w'].shape}")
    _check_quant(d["w"], "w")


def test_quant_exhaustive_bf16_sweep():
    """Rows enumerate every finite bf16 value below several amax values:
    normal, power-of-two, subnormal and the largest finite scale."""
    allv = all_finite_bf16()
    vals = oracle.bf16_bits_to_f32(allv)
    rows = []
    for amax_bits in (0x3F80, 0x4074, 0x43E0, 0x007F, 0x0001, 0x0080, 0x7F7F, 0x3C01,
                      0x42FE, 0x0010):
        amax = oracle.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0]
        sel = allv[np.abs(vals) <= amax]
        rows.append(np.concatenate([[amax_bits], sel]))
    K = max(len(r) for r in rows)
    K = (K + 15) // 16 * 16
    x = np.zeros((len(rows), K), np.uint16)
    for i, r in enumerate(rows):
        x[i, : len(r)] = r
    announce(f"quant exhaustive sweep {x.shape}")
    _check_quant(x, "act")


def test_quant_edge_rows():
    rng = np.random.default_rng(11)
    K = 96
    x = [np.zeros(K, np.uint16),                                   # all zero
         np.full(K, 0x8000, np.uint16),                            # all -0
         to_bf16_bits(rng.standard_normal(K) * 2.0**-130),         # subnormal scale
         to_bf16_bits(rng.standard_normal(K) * 1e30),
         to_bf16_bits(np.arange(K) - 48.0),
         to_bf16_bits(rng.standard_t(1.0, K))]
    x = np.stack(x)
    announce("quant edge rows")
    _check_quant(x, "act")


@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (3, 48, 64), (5, 1040, 1040), (7, 16400, 16400),
                                    (2, 20000, 20008), (129, 3072, 3080)])
def test_quant_ragged_and_strided(M, K, ld):
    rng = np.random.default_rng(M * 7 + K)
    full = random_bf16(rng, (M, ld))
    xd = dev_bf16(full)[:, :K]
    announce(f"quant ragged M={M} K={K} ld={ld}")
    q, s = w8.quant_act(xd)
    torch.cuda.synchronize()
    eq, es = oracle.quant_act(full[:, :K])
    assert_equal(host(s), es, "scale")
    assert_equal(host(q), eq, "q")


# ---------------------------------------------------------------- GEMM / linear

def _linear_case(x_bits, w_bits, bias_bits, ldx=None, ldo=None, check_ws=True):
    """Runs w8a8_linear and w8a8_scaled_mm and compares with the oracle."""
    M, K = x_bits.shape
    N = w_bits.shape[0]
    wq_e, sw_e = oracle.quantize_weights(w_bits)
    exp = oracle.linear(x_bits, wq_e, sw_e, bias_bits)

    wq, sw = w8.quantize_weights(dev_bf16(w_bits))
    if ldx is not None and ldx != K:
        xpad = np.zeros((M, ldx), np.uint16)
        xpad[:, :K] = x_bits
        xd = dev_bf16(xpad)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    bd = None if bias_bits is None else dev_bf16(bias_bits)
    if ldo is not None and ldo != N:
        out_full = torch.empty((M, ldo), dtype=torch.bfloat16, device="cuda")
        out = out_full[:, :N]
    else:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(w8.workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device="cuda")
    w8.linear(xd, wq, sw, bd, out=out, workspace=ws, acc_debug=acc)
    torch.cuda.synchronize()

    assert_equal(host(sw), sw_e, "w_scale")
    assert_equal(host(wq), wq_e, "wq")
    if check_ws:
        xq_d, sa_d = w8.workspace_views(ws, M, K)
        assert_equal(host(sa_d), exp["s_a"], "a_scale")
        assert_equal(host(xq_d), exp["xq"], "xq")
    assert_equal(host(acc), exp["acc"], "acc")
    stats = assert_bf16_close(host_bits(out), exp["y"])

    # the second op alone on the oracle's quantised activations
    if M > 0:
        out2 = w8.scaled_mm(dev(exp["xq"]), dev(exp["s_a"]), wq, sw, bd)
        acc2 = torch.empty((M, N), dtype=torch.int32, device="cuda")
        w8.scaled_mm(dev(exp["xq"]), dev(exp["s_a"]), wq, sw, bd, acc_debug=acc2)
        torch.cuda.synchronize()
        assert_equal(host(acc2), exp["acc"], "acc (scaled_mm)")
        assert_bf16_close(host_bits(out2), exp["y"])
    return stats, exp


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 48), (4, 100, 8192), (16, 70, 8192),
                                   (2, 129, 8208), (17, 33, 64), (33, 67, 80),
                                   (67, 17, 208), (16, 300, 112), (65, 129, 1040),
                                   (130, 260, 528), (257, 513, 256), (300, 700, 1296),
                                   (65, 33000, 1040), (127, 32776, 64)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_small_shapes(M, N, K, with_bias):
    rng = np.random.default_rng(M * 1000 + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    announce(f"linear small M={M} N={N} K={K} bias={with_bias} path={w8.linear_path(M, K, N)}")
    _linear_case(x, w, b)


@pytest.mark.parametrize("name", ["c1_64x256x128", "c2_512x4096x4096_outliers",
                                  "c3_512x4096x12288_student_t"])
def test_linear_probe_shapes(name):
    d = make_linear_inputs(name)
    announce(f"linear {name}")
    stats, exp = _linear_case(d["x"], d["w"], d["bias"])
    print(name, stats)


@pytest.mark.parametrize("name", ["dit_qkv_4352x3072x9216", "dit_out_4352x3072x3072",
                                  "dit_up_4352x3072x12288", "dit_down_4352x12288x3072"])
def test_linear_dit_full_size(name):
    d = make_linear_inputs(name)
    announce(f"linear full size {name}")
    stats, _ = _linear_case(d["x"], d["w"], d["bias"])
    print(name, stats)


@pytest.mark.parametrize("m", [1, 2, 8, 16, 17, 32])
def test_linear_modulation_full_size(m):
    d = make_linear_inputs(f"mod_m{m}_3072x18432")
    announce(f"linear modulation M={m} path={w8.linear_path(m, 3072, 18432)}")
    stats, _ = _linear_case(d["x"], d["w"], d["bias"])
    print(m, stats)


def test_linear_strided_x_and_out():
    rng = np.random.default_rng(21)
    for M in (5, 40):
        x = random_bf16(rng, (M, 256))
        w = random_bf16(rng, (72, 256), 0.02)
        announce(f"linear strided M={M}")
        _linear_case(x, w, None, ldx=264, ldo=75)


def test_small_m_and_gemm_paths_agree_per_row():
    """Row m gives the same xq, a_scale, acc and y at M = 16 (small-M kernel,
    two token blocks), M = 32 (small-M kernel, four token blocks) and M = 33
    (quantisation kernel + GEMM)."""
    d = make_linear_inputs("mod_m32_3072x18432")
    extra = random_bf16(np.random.default_rng(33), (1, 3072))
    x_all = np.concatenate([d["x"], extra])
    wq, sw = w8.quantize_weights(dev_bf16(d["w"]))
    bd = dev_bf16(d["bias"])
    res = {}
    for M in (16, 32, 33):
        assert w8.linear_path(M, 3072, 18432) == (w8.PATH_SMALL_M if M <= 32 else w8.PATH_GEMM)
        x = dev_bf16(x_all[:M])
        acc = torch.empty((M, 18432), dtype=torch.int32, device="cuda")
        ws = torch.empty((w8.workspace_bytes(M, 3072, 18432),), dtype=torch.uint8, device="cuda")
        announce(f"path agreement M={M}")
        y = w8.linear(x, wq, sw, bd, workspace=ws, acc_debug=acc)
        torch.cuda.synchronize()
        xq, sa = w8.workspace_views(ws, M, 3072)
        res[M] = [host(xq), host(sa), host(acc), host_bits(y)]
    for a, b, c in zip(res[16], res[32], res[33]):
        assert np.array_equal(a, b[:16])
        assert np.array_equal(b, c[:32])


def test_fused_qkv_equals_three_calls():
    rng = np.random.default_rng(31)
    M, K = 300, 512
    x = dev_bf16(random_bf16(rng, (M, K)))
    ws = [random_bf16(rng, (n, K), 0.02) for n in (192, 64, 64)]
    parts = [w8.quantize_weights(dev_bf16(w)) for w in ws]
    wq_f = torch.cat([p[0] for p in parts])
    sw_f = torch.cat([p[1] for p in parts])
    announce("fused QKV vs three calls")
    y_f = w8.linear(x, wq_f, sw_f)
    ys = [w8.linear(x, p[0], p[1]) for p in parts]
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_f), np.concatenate([host_bits(y) for y in ys], axis=1))


def test_deterministic_repeats():
    d = make_linear_inputs("c2_512x4096x4096_outliers")
    wq, sw = w8.quantize_weights(dev_bf16(d["w"]))
    x = dev_bf16(d["x"])
    announce("determinism")
    outs = [host_bits(w8.linear(x, wq, sw)) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_empty_m_is_noop():
    wq = torch.zeros((8, 64), dtype=torch.int8, device="cuda")
    sw = torch.ones((8,), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    y = w8.linear(x, wq, sw)
    xq, sa = w8.quant_act(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 8) and xq.shape == (0, 64) and sa.shape == (0,)


def test_extreme_accumulators():
    """All +-127 operands reach |acc| = 127^2 K without overflow."""
    M, N, K = 20, 36, 16384
    x = np.full((M, K), 0x3F80, np.uint16)          # 1.0
    x[1::2] = 0xBF80                                # -1.0
    w = np.full((N, K), 0x3F80, np.uint16)
    announce("extreme accumulators")
    _linear_case(x, w, None)


def test_linear_subnormal_scales_and_outputs():
    """Weights ~1e-41 (bf16 subnormals) give subnormal fp32 weight scales
    (exact-division quantisation path) and bf16-subnormal outputs, on both
    the small-M kernel and the GEMM."""
    rng = np.random.default_rng(41)
    K, N = 512, 320
    w = to_bf16_bits(rng.normal(0.0, 1e-41, (N, K)))
    assert np.any((w & 0x7F80) == 0) and np.any(w & 0x7FFF)
    for M in (3, 70):
        x = random_bf16(rng, (M, K))
        announce(f"subnormal scales/outputs M={M}")
        _, exp = _linear_case(x, w, None)
        y = oracle.bf16_bits_to_f32(exp["y"])
        assert np.any((np.abs(y) > 0) & (np.abs(y) < np.finfo(np.float32).tiny))


@pytest.mark.parametrize("M,N,K", [(4, 70, 1040), (5, 70, 1040), (8, 70, 1040), (9, 70, 1040),
                                   (12, 18432, 3072), (16, 200, 3072), (6, 70, 3088), (13, 18432, 3072),
                                   (17, 70, 1040), (25, 200, 3072), (32, 18432, 3072),
                                   (24, 70, 3088), (32, 33, 4096)])
def test_linear_small_m_work_splits(M, N, K):
    """Every way the small-M kernel splits the activation rows over its waves
    (W = 4 waves for N = 33, 70 and 200 and 9 for N = 18432 up to M = 8, 12
    from M = 9 on): one row per wave (M <= W), two rows per wave held across
    the weight requests (W < M <= 16), rows quantised before the stream
    (every M above 16; fp16 above W, in the fp16 tests) and rows longer than
    the register-resident limit (K > 3072)."""
    rng = np.random.default_rng(M * 31 + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01)
    announce(f"small-M work split M={M} N={N} K={K}")
    assert w8.linear_path(M, K, N) == w8.PATH_SMALL_M
    print(_linear_case(x, w, b)[0])


@pytest.mark.parametrize("N", [2056, 2052, 2050])
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_256_tile_store_paths(N, with_bias):
    """The 256x256 tile with each output store path: 16-byte rows staged in
    LDS (N % 8 == 0), 8-byte stores (N % 4 == 0) and 2-byte stores, with and
    without bias."""
    M, K = 4352, 272
    assert w8.gemm_tile(M, K, N) == (256, 256)
    rng = np.random.default_rng(N * 3 + with_bias)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    announce(f"256 tile store path M={M} N={N} K={K} bias={with_bias}")
    print(_linear_case(x, w, b)[0])


# Split K: shapes whose 256x256 tiles fill at most half of the compute units
# or whose 128x128 tiles fill at most one round (K split in two), and skinny
# shapes on 64x64 tiles (K split in up to four); w8a8_linear then splits K
# (its workspace holds the partial sums), w8a8_scaled_mm does not. Both must
# give the oracle's acc and the same y bits. (K = 1040 / 2064: the last split
# ends on a 16-byte tail.)
@pytest.mark.parametrize("M,N,K,with_bias", [(512, 12288, 4096, True), (700, 8200, 2000, True),
                                             (520, 10240, 1040, False), (512, 4096, 4096, False),
                                             (200, 2056, 1040, True), (1024, 2056, 2064, True),
                                             (64, 18432, 3072, True), (40, 1032, 2064, True),
                                             (100, 2056, 4096, False), (100, 18432, 3072, True)])
def test_linear_split_k(M, N, K, with_bias):
    assert w8.workspace_bytes(M, K, N) > M * K + 4 * M + 512, "the split path is taken"
    rng = np.random.default_rng(M + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    announce(f"split-K linear M={M} N={N} K={K} bias={with_bias}")
    _, exp = _linear_case(x, w, b)
    wq, sw = w8.quantize_weights(dev_bf16(w))
    bd = None if b is None else dev_bf16(b)
    y_split = w8.linear(dev_bf16(x), wq, sw, bd)
    y_one = w8.scaled_mm(dev(exp["xq"]), dev(exp["s_a"]), wq, sw, bd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_split), host_bits(y_one))


def test_linear_split_k_fallback_on_unaligned_output():
    """An output row stride that is not a multiple of 8 takes the one-pass GEMM."""
    M, N, K = 512, 12288, 2048
    rng = np.random.default_rng(5)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    announce("split-K shape, output stride N + 4")
    _linear_case(x, w, None, ldo=N + 4)
