"""GPU parity of the producers fused with the activation quantisation
(w8a8_layernorm_modulate_quant_act, w8a8_gelu_quant_act) against the oracle.

The LayerNorm's bf16 row y comes from an fp32 evaluation in the kernel, GELU's
from the library's built-in table (GELU in double precision, rounded once to
bf16), and both from a float64 evaluation in the oracle, so y is checked
against the oracle's exact value v: |y - v| must stay within half a bf16 ulp
plus the fp32 error bound the oracle derives
(oracle.layernorm_modulate_err_bound with the kernel's summation depth
K / 64 + 16, oracle.gelu_err_bound). Where y is not the
nearest bf16 to v it can only be the other neighbour, and only within that
bound of a midpoint; the count of such elements is reported. The int8 codes
and scales are then checked bit for bit against the oracle's quantisation
of the kernel's own y, so both sides take every integer decision on the same
bf16 values.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, assert_equal, dev_bf16, host, host_bits
from synth_inputs import all_finite_bf16, random_bf16, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _depth(K):
    return K // 64 + 16


def check(v, bound, y_bits, xq, sa) -> dict:
    ok = oracle.bf16_within(y_bits, v, bound)
    assert ok.all(), (np.argwhere(~ok)[:5], v[~ok][:5], y_bits[~ok][:5])
    q_e, s_e = oracle.quant_act(y_bits)
    assert_equal(xq, q_e, "xq")
    assert_equal(sa, s_e, "a_scale")
    nearest = oracle.f64_to_bf16_bits(v)
    st = {"n": int(v.size), "n_not_nearest": int(np.count_nonzero(y_bits != nearest))}
    print(f"  {st}", flush=True)
    return st


def _pad(bits, ld):
    if ld is None:
        return dev_bf16(bits)
    M, K = bits.shape
    p = np.zeros((M, ld), np.uint16)
    p[:, :K] = bits
    return dev_bf16(p)[:, :K]


def run_ln(x, sh, sc, eps, rpg=None, ldx=None, mod_ld=None):
    """Runs the fused LayerNorm twice (with and without y) and checks it."""
    M, K = x.shape
    G = sh.shape[0]
    xd = _pad(x, ldx)
    if mod_ld is not None:       # shift and scale as chunks of one [G, mod_ld] buffer
        buf = np.zeros((G, mod_ld), np.uint16)
        buf[:, :K] = sh
        buf[:, mod_ld - K:] = sc
        bd = dev_bf16(buf)
        shd, scd = bd[:, :K], bd[:, mod_ld - K:]
    else:
        shd, scd = dev_bf16(sh), dev_bf16(sc)
    announce(f"layernorm_modulate M={M} K={K} G={G} rpg={rpg} ldx={ldx} mod_ld={mod_ld}")
    xq, sa, y = w8.layernorm_modulate_quant_act(xd, shd, scd, eps, rows_per_group=rpg,
                                                return_y=True)
    xq2, sa2 = w8.layernorm_modulate_quant_act(xd, shd, scd, eps, rows_per_group=rpg)
    torch.cuda.synchronize()
    xq, sa, y = host(xq), host(sa), host_bits(y)
    assert_equal(host(xq2), xq, "xq without y")
    assert_equal(host(sa2), sa, "a_scale without y")
    v = oracle.layernorm_modulate(x, sh, sc, eps, rows_per_group=rpg)
    bound = oracle.layernorm_modulate_err_bound(x, sh, sc, eps, rows_per_group=rpg,
                                                depth=_depth(K))
    return check(v, bound, y, xq, sa)


def run_gelu(z, approximate, ldz=None):
    M, K = z.shape
    zd = _pad(z, ldz)
    announce(f"gelu {approximate} M={M} K={K} ldz={ldz}")
    xq, sa, y = w8.gelu_quant_act(zd, approximate, return_y=True)
    xq2, sa2 = w8.gelu_quant_act(zd, approximate)
    torch.cuda.synchronize()
    xq, sa, y = host(xq), host(sa), host_bits(y)
    assert_equal(host(xq2), xq, "xq without y")
    assert_equal(host(sa2), sa, "a_scale without y")
    v = oracle.gelu(z, approximate)
    return check(v, oracle.gelu_err_bound(z, approximate), y, xq, sa)


def _ln_inputs(M, K, G=1, seed=0, outliers=0):
    rng = np.random.default_rng(seed + 31 * M + K)
    x = random_bf16(rng, (M, K), 1.0)
    if outliers:
        cols = rng.choice(K, outliers, replace=False)
        x[:, cols] = random_bf16(rng, (M, outliers), 30.0)
    return x, random_bf16(rng, (G, K), 0.5), random_bf16(rng, (G, K), 0.5)


# every launch configuration (1 to 4 waves per row, 1..8 chunks per lane),
# ragged K and partial last workgroups; rows of 2049-3072 elements take three
# waves per row up to 1024 rows and two beyond
LN_SHAPES = [(1, 16), (3, 48), (5, 512), (7, 528), (4, 1024), (9, 1040), (6, 2048), (3, 2064),
             (10, 3072), (1023, 3072), (1024, 2064), (1025, 3072), (2, 4096), (5, 4112),
             (3, 8192), (6, 12288), (2, 12304), (3, 16384)]


@pytest.mark.parametrize("M,K", LN_SHAPES)
def test_layernorm_shapes(M, K):
    x, sh, sc = _ln_inputs(M, K, outliers=max(1, K // 200))
    st = run_ln(x, sh, sc, 1e-6)
    assert st["n_not_nearest"] <= max(2, st["n"] // 200), st


def test_layernorm_grouped_strided():
    """Two samples' tokens, shift and scale as chunks of one modulation
    output with row stride 6K (as a DiT's [B, 6 * hidden] modulation gives),
    padded x rows."""
    x, sh, sc = _ln_inputs(37, 3072, G=3, seed=3, outliers=15)
    run_ln(x, sh, sc, 1e-6, rpg=13, ldx=3080, mod_ld=6 * 3072)
    x, sh, sc = _ln_inputs(5, 512, G=5, seed=4)
    run_ln(x, sh, sc, 1e-5, rpg=1, mod_ld=1024)


def test_layernorm_edge_rows():
    K = 3072
    rng = np.random.default_rng(9)
    x, sh, sc = _ln_inputs(8, K, seed=9)
    x[0] = to_bf16_bits(np.full(K, 5.0))                       # constant: x - mean = 0
    x[1] = 0                                                   # all zero
    x[2] = to_bf16_bits(rng.standard_normal(K) * 1e-3)
    x[3] = to_bf16_bits(rng.standard_normal(K) * 1e4)
    x[4] = to_bf16_bits(rng.standard_normal(K) * 1e-39)        # bf16 subnormals
    x[5] = to_bf16_bits(rng.standard_normal(K) + 7.0)          # mean far from zero
    x[6, ::2] = 0x3F80                                          # +-1 alternating
    x[6, 1::2] = 0xBF80
    sc[0, :] = to_bf16_bits(np.full(K, -1.0))                  # 1 + scale = 0
    run_ln(x, sh, sc, 1e-6)
    # zero shift: the constant and zero rows give an all-zero y (scale 0)
    zero = np.zeros_like(sh)
    st = run_ln(x[:2], zero, sc, 1e-6)
    assert st["n_not_nearest"] == 0


def test_layernorm_eps_matters():
    x = to_bf16_bits(np.tile([1e-3, -1e-3], (4, 256)))
    sh, sc = np.zeros((1, 512), np.uint16), np.zeros((1, 512), np.uint16)
    for eps in (1e-6, 1e-2, 1.0):
        run_ln(x, sh, sc, eps)


def test_layernorm_ldy():
    """y written with its own row stride through the C ABI."""
    M, K, ldy = 6, 1040, 1056
    x, sh, sc = _ln_inputs(M, K, seed=7)
    xd, shd, scd = dev_bf16(x), dev_bf16(sh), dev_bf16(sc)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    yb = torch.full((M, ldy), 12345, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    announce(f"layernorm_modulate ldy={ldy}")
    st = w8.lib().w8a8_layernorm_modulate_quant_act(
        ctypes.c_void_p(xd.data_ptr()), M, K, K, ctypes.c_void_p(shd.data_ptr()),
        ctypes.c_void_p(scd.data_ptr()), K, M, ctypes.c_float(1e-6),
        ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sa.data_ptr()),
        ctypes.c_void_p(yb.data_ptr()), ldy, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == w8.OK
    torch.cuda.synchronize()
    y = host_bits(yb)
    assert (y[:, K:] == 12345).all(), "nothing written past K"
    v = oracle.layernorm_modulate(x, sh, sc, 1e-6)
    check(v, oracle.layernorm_modulate_err_bound(x, sh, sc, 1e-6, depth=_depth(K)),
          np.ascontiguousarray(y[:, :K]), host(xq), host(sa))


def test_layernorm_full_dit_rows():
    """The DiT block's LayerNorm input at full size: 4352 tokens x 3072."""
    x, sh, sc = _ln_inputs(4352, 3072, seed=1, outliers=15)
    st = run_ln(x, sh, sc, 1e-6)
    assert st["n_not_nearest"] <= st["n"] // 1000, st


# --- GELU ---------------------------------------------------------------

GELU_SHAPES = [(1, 16), (5, 528), (3, 3072), (2, 4112), (3, 12288), (2, 12304), (2, 24576),
               (1, 32768)]


@pytest.mark.parametrize("approximate", ["none", "tanh"])
@pytest.mark.parametrize("M,K", GELU_SHAPES)
def test_gelu_shapes(approximate, M, K):
    rng = np.random.default_rng(M * 13 + K)
    z = random_bf16(rng, (M, K), 1.0)
    z[:, rng.choice(K, max(1, K // 200), replace=False)] *= 0          # exact zeros
    st = run_gelu(z, approximate)
    assert st["n_not_nearest"] <= max(2, st["n"] // 1000), st


@pytest.mark.parametrize("approximate", ["none", "tanh"])
@pytest.mark.parametrize("K", [16, 4080])
def test_gelu_every_bf16_value(approximate, K):
    """Every finite bf16 z, in rows of 16 (scales from neighbours of similar
    size) and of 4080 values."""
    z = all_finite_bf16()
    z = z[: z.size // K * K].reshape(-1, K)
    st = run_gelu(z, approximate)
    assert st["n_not_nearest"] <= st["n"] // 1000, st


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_strided(approximate):
    rng = np.random.default_rng(3)
    run_gelu(random_bf16(rng, (9, 1040), 2.0), approximate, ldz=1056)


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_full_dit_rows(approximate):
    """The FFN-down input at full size: 4352 tokens x 12288."""
    rng = np.random.default_rng(2)
    z = random_bf16(rng, (4352, 12288), 1.0)
    st = run_gelu(z, approximate)
    assert st["n_not_nearest"] <= st["n"] // 1000, st


# Every GELU call looks its elements up in the built-in bf16 -> bf16 table
# (computed at build time in double precision, rounded once to bf16).


@pytest.fixture(scope="module")
def host_tables(tmp_path_factory):
    """The tables as the library's own generator writes them (g++ on the host)."""
    import re
    import shutil
    if shutil.which("g++") is None:
        pytest.skip("needs g++ to build the table generator")
    from w8a8_int8_dynamic_quant_amd import build_lib
    out = build_lib.gen_gelu_table(build_dir=str(tmp_path_factory.mktemp("gelu_tab")))
    vals = [int(v, 16) for v in re.findall(r"0x([0-9a-f]{4}),", open(out).read())]
    return np.array(vals, np.uint16).reshape(2, 65536)


@pytest.mark.parametrize("form,approximate", [(0, "none"), (1, "tanh")])
def test_gelu_every_bf16_value_is_the_table_entry(host_tables, form, approximate):
    """Every finite bf16 z, in 1040 rows of 4080 (each row 255 values, 16
    times): y is exactly the table's entry for z, the same bits in every row
    that holds z, and xq / a_scale are the quantisation of those rows."""
    z = all_finite_bf16().reshape(16, 4080)
    big = np.tile(z, (65, 1))
    st = run_gelu(big, approximate)
    assert st["n_not_nearest"] <= 2, st
    announce(f"gelu {approximate} against the host table")
    xq, sa, y = w8.gelu_quant_act(dev_bf16(big), approximate, return_y=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_tables[form][big])
    q_e, s_e = oracle.quant_act(host_tables[form][big])
    assert_equal(host(xq), q_e, "xq")
    assert_equal(host(sa), s_e, "a_scale")


@pytest.mark.parametrize("approximate", ["none", "tanh"])
@pytest.mark.parametrize("M,K", [(1100, 4112), (262160, 16), (400, 12288), (3001, 1552),
                                 (520, 8192), (300, 16384), (260, 16400), (180, 24576),
                                 (130, 32768), (600, 24576),
                                 # sixteen waves per row (at most 512 rows of at most
                                 # 16384 elements), over one and two sweeps of the grid,
                                 # and four waves just past 512 rows
                                 (512, 3088), (340, 12304), (512, 16384), (513, 3072)])
def test_gelu_table_path_shapes(approximate, M, K):
    """Ragged K (past-K chunks in a lane's last slots), one to eight chunks
    per lane on four waves per row up to K = 16384 (more than 512 rows),
    sixteen waves per row (at most 512 rows), eight waves per row beyond
    K = 16384 (K = 16400, 24576, 32768), and more rows than the grid takes
    in one pass (1100 x 4112, 600 x 24576, 340 x 12304, 512 x 16384)."""
    rng = np.random.default_rng(M + K)
    st = run_gelu(random_bf16(rng, (M, K), 1.5), approximate)
    assert st["n_not_nearest"] <= max(2, st["n"] // 1000), st


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_table_path_strided(approximate):
    rng = np.random.default_rng(5)
    run_gelu(random_bf16(rng, (2100, 2048), 1.0), approximate, ldz=2056)


def test_gelu_table_path_two_streams():
    """Table-path calls of the same form on two streams at once rebuild the
    shared table with the same bytes: each result matches its one-stream run."""
    rng = np.random.default_rng(17)
    z1, z2 = random_bf16(rng, (1100, 4096), 1.0), random_bf16(rng, (1100, 4096), 2.0)
    d1, d2 = dev_bf16(z1), dev_bf16(z2)
    announce("gelu table path, two streams")
    ref = [w8.gelu_quant_act(d, "none", return_y=True) for d in (d1, d2)]
    torch.cuda.synchronize()
    ref = [tuple(host_bits(t) if t.dtype == torch.bfloat16 else host(t) for t in r) for r in ref]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        with torch.cuda.stream(s1):
            a = w8.gelu_quant_act(d1, "none", return_y=True)
        with torch.cuda.stream(s2):
            b = w8.gelu_quant_act(d2, "none", return_y=True)
        torch.cuda.synchronize()
        for got, exp in ((a, ref[0]), (b, ref[1])):
            assert np.array_equal(host(got[0]), exp[0])
            assert np.array_equal(host(got[1]), exp[1])
            assert np.array_equal(host_bits(got[2]), exp[2])


# --- with the GEMM ----------------------------------------------------------

@pytest.mark.parametrize("producer", ["layernorm", "gelu"])
def test_fused_producer_feeds_the_gemm(producer):
    """Producer codes + scaled_mm give the same bits as linear() on the
    producer's own bf16 output (the unfused path)."""
    M, K, N = 300, 3072, 520
    rng = np.random.default_rng(21)
    x = random_bf16(rng, (M, K), 1.0)
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01)
    wq, sw = w8.quantize_weights(dev_bf16(w))
    bias = dev_bf16(b)
    announce(f"fused {producer} + scaled_mm M={M} K={K} N={N}")
    if producer == "layernorm":
        sh, sc = random_bf16(rng, (1, K), 0.5), random_bf16(rng, (1, K), 0.5)
        xq, sa, y = w8.layernorm_modulate_quant_act(dev_bf16(x), dev_bf16(sh), dev_bf16(sc),
                                                    return_y=True)
    else:
        xq, sa, y = w8.gelu_quant_act(dev_bf16(x), "tanh", return_y=True)
    fused = w8.scaled_mm(xq, sa, wq, sw, bias)
    unfused = w8.linear(y, wq, sw, bias)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(fused), host_bits(unfused))
