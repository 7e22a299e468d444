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
                                    (2, 20000, 20008), (129, 3072, 3080),
                                    # three and four waves per row, ragged rows and
                                    # partial last workgroups
                                    (3, 2064, 2072), (5, 3056, 3056), (2, 3088, 3096),
                                    (7, 4096, 4104), (1025, 4080, 4080),
                                    # one workgroup of eight waves per row, 2 to 8 chunks
                                    # per thread, and four waves (4 chunks) for rows of
                                    # 4112-8192 elements beyond 2048 rows
                                    (3, 4112, 4120), (5, 8192, 8192), (3, 14000, 14000),
                                    (2, 24592, 24600), (3, 32768, 32768), (2049, 4112, 4120),
                                    (2050, 8192, 8192)])
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
        # the padding holds 65536.0: read into any row's amax, it would
        # change that row's scale and every code
        xpad = np.full((M, ldx), 0x4780, np.uint16)
        xpad[:, :K] = x_bits
        xd = dev_bf16(xpad)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    bd = None if bias_bits is None else dev_bf16(bias_bits)
    out_full = None
    if ldo is not None and ldo != N:
        # a sentinel in the output's padding columns, checked after the call
        out_full = dev_bf16(np.full((M, ldo), 0x1234, np.uint16))
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
    if out_full is not None:
        assert (host_bits(out_full)[:, N:] == 0x1234).all(), "output padding written"

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
                                   (40, 72, 4112), (20, 40, 8192), (3, 40, 24592),
                                   (2, 24, 32768),
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


@pytest.mark.parametrize("M,K,ldx", [(5, 256, 264), (40, 256, 264), (12, 256, 264), (20, 256, 264),
                                     (3, 3088, 3096)])
def test_linear_strided_x_and_out(M, K, ldx):
    """Row strides of x and out that differ from K and N, on the small-M row
    modes (M = 5), the split kernel's LDS-staged rows (M = 12, 20) and
    two-pass long rows (K = 3088), and the GEMM path (M = 40)."""
    rng = np.random.default_rng(21 + M)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (72, K), 0.02)
    announce(f"linear strided M={M} K={K} ldx={ldx}")
    _linear_case(x, w, None, ldx=ldx, ldo=75)


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


# the largest K the library accepts: a multiple of 16 with 127^2 K < 2^31
K_LARGEST = (w8.K_MAX // 16) * 16


def _signed_ones(R, K):
    """Rows of +1.0 (even rows) and -1.0 (odd rows): every code is +-127."""
    x = np.full((R, K), 0x3F80, np.uint16)
    x[1::2] = 0xBF80
    return x


@pytest.mark.parametrize("M,N", [(3, 40), (130, 72)])
def test_linear_largest_k_extreme_accumulators(M, N):
    """At the largest accepted K, +-127 codes throughout give |acc| =
    127^2 K, the int32 limit the K bound is set by, with both signs: the
    GEMM split in K on 64x64 tiles (M = 3) and on 128x128 tiles (M = 130),
    against the oracle on every output."""
    x, w = _signed_ones(M, K_LARGEST), _signed_ones(N, K_LARGEST)
    announce(f"largest K M={M} N={N} K={K_LARGEST} tile={w8.gemm_tile(M, K_LARGEST, N)}")
    _, exp = _linear_case(x, w, None)
    assert np.abs(exp["acc"]).max() == 127 * 127 * K_LARGEST < 2**31


@pytest.mark.parametrize("M,N", [(4352, 3072), (2048, 4096)])
def test_linear_largest_k_256_tiles(M, N):
    """The 256x256-tile kernel at the largest accepted K, whole tiles
    (4352 x 3072: 204 tiles) and 128-row halves (2048 x 4096: 128 tiles),
    with +-127 codes throughout. Row m of x and row n of W are +-1.0 by the
    parity of m and n, so every output is one of four values. Quantisation
    is per row and per output channel, so the oracle run on rows 0-1 of x
    and W gives those four values exactly; every element of xq, a_scale,
    acc and y is compared with them."""
    K = K_LARGEST
    assert w8.gemm_tile(M, K, N) == (256, 256)
    x, w = _signed_ones(M, K), _signed_ones(N, K)
    wq_e, sw_e = oracle.quantize_weights(w[:2])
    exp = oracle.linear(x[:2], wq_e, sw_e, None)
    assert np.abs(exp["acc"]).max() == 127 * 127 * K

    wq, sw = w8.quantize_weights(dev_bf16(w))
    del w
    xd = dev_bf16(x)
    del x
    ws = torch.empty((w8.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    announce(f"largest K, 256x256 tiles M={M} N={N} K={K}")
    y = w8.linear(xd, wq, sw, workspace=ws, acc_debug=acc)
    torch.cuda.synchronize()

    # the codes, on the device (M x K bytes): rows alternate the oracle's two
    xq_d, sa_d = w8.workspace_views(ws, M, K)
    for p in (0, 1):
        assert torch.equal(xq_d[p::2], dev(exp["xq"][p]).expand(M // 2, K)), f"xq rows {p}::2"
        assert torch.equal(wq[p::2], dev(wq_e[p]).expand(N // 2, K)), f"wq rows {p}::2"
    assert_equal(host(sa_d), np.tile(exp["s_a"], M // 2), "a_scale")
    assert_equal(host(sw), np.tile(sw_e, N // 2), "w_scale")
    assert_equal(host(acc), np.tile(exp["acc"], (M // 2, N // 2)), "acc")
    assert_bf16_close(host_bits(y), np.tile(exp["y"], (M // 2, N // 2)))
    del xd, ws, acc, y, wq
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K", [(5, 72, 256), (130, 72, 256), (2048, 4096, 256),
                                   (4352, 3072, 256)])
def test_linear_largest_output_stride(M, N, K):
    """Output rows W8A8_LDO_MAX elements apart, the largest stride accepted
    (the byte offsets within a 256-row tile stay below 2^32), on the
    small-M kernel (M = 5), 128x128 tiles (M = 130) and 256x256 tiles as
    halves (2048 x 4096) and whole (4352 x 3072): every output against the
    oracle, and the columns beside the output and at the end of every row
    left as they were."""
    rng = np.random.default_rng(91 + M)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    wq_e, sw_e = oracle.quantize_weights(w)
    exp = oracle.linear(x, wq_e, sw_e, None)
    wq, sw = w8.quantize_weights(dev_bf16(w))
    ldo = w8.LDO_MAX
    out_full = torch.full((M, ldo), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    announce(f"largest output stride M={M} N={N} K={K} ldo={ldo} "
             f"path={w8.linear_path(M, K, N)} tile={w8.gemm_tile(M, K, N)}")
    w8.linear(dev_bf16(x), wq, sw, out=out_full[:, :N])
    torch.cuda.synchronize()
    assert_bf16_close(host_bits(out_full[:, :N]), exp["y"])
    pad = torch.cat([out_full[:, N:N + 256], out_full[:, ldo - 256:]], dim=1)
    assert (host_bits(pad) == 0x1234).all(), "output padding written"
    del out_full, pad
    torch.cuda.empty_cache()


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


def _small_m_form(M, K, N, cus=256):
    """Which small-M kernel form serves (M, K, N) on a 256-CU device, by the
    launcher's rule: the weight waves G = clamp(ceil(ceil(N/8) / cus), 4, 12);
    the quantiser waves H (one per row up to 4 rows, else a multiple of 4 that
    fits beside G in 16 waves, at most M); the split kernel for K > 3072 or
    above 8 rows with at most three rows per quantiser, the row modes
    otherwise. Split: the weight stream whole or refilled (more windows than
    24, 16 or 12 for 1-2, 3 or 4 token blocks), and the quantisers' rows
    staged in LDS (when 8 TB slots of 256 ceil(K/128) + 32 bytes fit in
    159 KiB; above K = 3072 quantised in two passes over LDS), else in
    registers (K <= 3072) or read twice from memory."""
    G = min(12, max(4, -(-(-(-N // 8)) // cus)))
    H = M if M <= 4 else min(M, 4 * min(-(-M // 4), (16 - G) // 4))
    TB = -(-M // 8)
    if K > 3072 or (M > 8 and -(-M // H) <= 3):
        depth = {1: 24, 2: 24, 3: 16, 4: 12}[TB]
        stream = "refill" if K > 128 * depth else "whole"
        nwin = -(-K // 128)
        if 8 * TB * (256 * nwin + 32) <= 159 * 1024:
            rows = "staged" if K <= 3072 else "staged long"
        else:
            rows = "two-pass" if K > 3072 else "registers"
        return "split", stream, rows, TB
    W = 12 if TB >= 2 else G
    return "rows", ("one" if M <= W and TB == 1 else "three" if TB == 4 else "two"), TB


_WORK_SPLITS = [(4, 70, 1040), (5, 70, 1040), (8, 70, 1040), (9, 70, 1040), (12, 18432, 3072),
                (16, 200, 3072), (3, 72, 4112), (6, 70, 3088), (10, 72, 5136), (13, 18432, 3072),
                (17, 70, 1040), (20, 200, 3072), (20, 18432, 2048), (25, 200, 3072), (26, 70, 2048),
                (28, 70, 1040), (32, 18432, 3072), (24, 70, 3088), (32, 33, 4096),
                # the largest LDS staging (156.7 of 159 KiB), the next K in registers,
                # and three token blocks staged at K = 3072 (148 KiB)
                (26, 70, 2432), (26, 70, 2448), (24, 70, 3072),
                # long rows staged at the LDS limit (two token blocks, K = 4992;
                # one, K = 8192), the next K read twice from memory, and three
                # token blocks read twice
                (16, 72, 4992), (16, 72, 5008), (8, 72, 8192), (20, 72, 4096),
                # long rows take down to one weight wave per workgroup: two here,
                # the last workgroup's second one past N
                (2, 2056, 4112)]


def test_small_m_work_splits_cover_every_form():
    """The parity cases below reach every form of both small-M kernels."""
    forms = {_small_m_form(M, K, N) for (M, N, K) in _WORK_SPLITS}
    want = {("rows", "one", 1), ("rows", "two", 1), ("rows", "two", 2), ("rows", "two", 3),
            ("rows", "three", 4)}
    want |= {("split", "refill", "two-pass", tb) for tb in (2, 3, 4)}
    want |= {("split", "refill", "staged long", tb) for tb in (1, 2, 3)}
    want |= {("split", "whole", "staged", tb) for tb in (2, 3, 4)}
    want |= {("split", "refill", "staged", tb) for tb in (3, 4)}
    want |= {("split", "refill", "registers", 4)}
    assert want <= forms, want - forms


@pytest.mark.parametrize("M,N,K", _WORK_SPLITS)
def test_linear_small_m_work_splits(M, N, K):
    """Every form of the two small-M kernels (test above): row modes, where
    each wave holds one, two or three rows in registers across its first
    weight requests (W = 4 waves for N = 33, 70, 72 and 200 and 9 for
    N = 18432 up to M = 8, 12 from M = 9 on); split roles, where quantiser
    waves without weight rows quantise rows staged in LDS, held in
    registers or read twice from memory while the weight waves stream, with
    all of a row group's windows in flight or refilled as consumed."""
    rng = np.random.default_rng(M * 31 + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01)
    announce(f"small-M work split M={M} N={N} K={K} form={_small_m_form(M, K, N)}")
    assert w8.linear_path(M, K, N) == w8.PATH_SMALL_M
    print(_linear_case(x, w, b)[0])


def _tie_rows(rng, M, K):
    """bf16 rows whose quantisation meets rounding ties: amax 127 * 2^e gives
    the scale 2^e exactly, so every x = (k + 1/2) 2^e (|k + 1/2| <= 62.5,
    seven significant bits, exact in bf16) has x / s exactly half-way between
    two codes (round half to even decides); rows with a subnormal scale
    (every element takes the division); and plain rows between them."""
    rows = []
    for r in range(M):
        kind = r % 3
        if kind == 0:
            e = int(rng.integers(-10, 10))
            v = (rng.integers(-63, 63, K) + 0.5) * 2.0 ** e
            v[int(rng.integers(0, K))] = 127.0 * 2.0 ** e * (1 if rng.random() < 0.5 else -1)
        elif kind == 1:
            v = rng.standard_normal(K) * 2.0 ** -133
        else:
            v = rng.standard_normal(K)
        rows.append(to_bf16_bits(v))
    return np.stack(rows)


@pytest.mark.parametrize("M,N,K", [(1, 72, 3072), (5, 72, 3072), (13, 18432, 1024),
                                   (32, 18432, 1024), (12, 200, 3072), (16, 200, 3072),
                                   (20, 200, 3072), (30, 200, 3072), (9, 200, 4112),
                                   (17, 72, 4096)])
def test_linear_small_m_rounding_ties(M, N, K):
    """The fused small-M kernels' on-chip quantisation on rows full of exact
    rounding ties and on rows with subnormal scales, in each way they hold the
    rows (row modes: one, two, three per wave; split roles: staged in LDS,
    in registers, read twice from memory): codes and scales bit-exact
    against the oracle (which rounds fl32(x / s) half to even)."""
    assert w8.linear_path(M, K, N) == w8.PATH_SMALL_M
    rng = np.random.default_rng(M * 101 + K)
    x = _tie_rows(rng, M, K)
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01)
    announce(f"small-M rounding ties M={M} N={N} K={K}")
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


def _pp_halves(M, N):
    """True when the 256x256 kernel runs some tiles as 128-row halves (the
    rule the launcher applies, per XCD of cus/8 compute units: every tile
    when the XCD's tiles fill at most half of them, else the tiles beyond
    whole rounds when they fill at most half a round)."""
    cpx = torch.cuda.get_device_properties(0).multi_processor_count // 8
    T = -(-M // 256) * -(-N // 256)
    for x in range(8):
        tx = T // 8 + (1 if x < T % 8 else 0)
        if 0 < tx and 2 * tx <= cpx:
            return True
        rem = tx % cpx if tx > cpx else 0
        if 0 < rem and 2 * rem <= cpx:
            return True
    return False


@pytest.mark.parametrize("M,N,K,with_bias", [(4152, 9224, 272, True), (4100, 9218, 272, False),
                                             (4352, 9220, 1040, True), (4352, 12288, 208, False),
                                             (512, 12288, 4096, True), (700, 8200, 2000, True),
                                             (520, 10240, 1040, False), (516, 8196, 528, True),
                                             (516, 8194, 528, False)])
def test_linear_256_tile_halves(M, N, K, with_bias):
    """Tiles split into 128-row halves: in the last round (the 4352-row
    shapes: a last M tile whose second half is empty (4100: 4 rows in the
    first) or ragged (4152), the three store paths (N % 8 == 0, N % 4 == 0,
    else) and a K tail), and every tile of shapes whose tiles fill at most
    half of the compute units (M = 516: a last M tile of 4 rows, whose second
    half is empty; N % 8 == 4 and N % 4 == 2)."""
    assert w8.gemm_tile(M, K, N) == (256, 256)
    assert _pp_halves(M, N)
    rng = np.random.default_rng(M + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    announce(f"256 tile halves M={M} N={N} K={K} bias={with_bias}")
    print(_linear_case(x, w, b)[0])


# Split K: shapes whose 128x128 tiles fill at most one round (K split in
# two), and skinny shapes on 64x64 tiles (K split in up to four);
# w8a8_linear then splits K (its workspace holds the partial sums),
# w8a8_scaled_mm does not. Both must give the oracle's acc and the same y
# bits. (K = 1040 / 2064: the last split ends on a 16-byte tail.)
@pytest.mark.parametrize("M,N,K,with_bias", [(512, 4096, 4096, False),
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
    """An output row stride that is not a multiple of 8 takes the one-pass GEMM
    (a shape whose 128x128 tiles split K otherwise)."""
    M, N, K = 512, 4096, 2048
    rng = np.random.default_rng(5)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    announce("split-K shape, output stride N + 4")
    _linear_case(x, w, None, ldo=N + 4)
