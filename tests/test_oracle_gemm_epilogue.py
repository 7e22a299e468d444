"""Pins of the oracle's integer product and scale epilogue (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_arith import f32_add, f32_mul, to_bf16_bits as exact_bf16, to_f32
from golden_io import epilogue_cases, gemm_case
from synth_inputs import to_bf16_bits


def test_gemm_hand_case():
    xq, wq, acc = gemm_case()
    got = oracle.gemm_exact(np.array(xq, np.int8), np.array(wq, np.int8))
    assert got.dtype == np.int32
    assert got.tolist() == acc


def _brute(xq, wq):
    M, K = len(xq), len(xq[0])
    N = len(wq)
    return [[sum(int(xq[m][k]) * int(wq[n][k]) for k in range(K)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (7, 2, 13), (9, 11, 33),
                                   (4, 6, 64)])
def test_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    exp = _brute(xq.tolist(), wq.tolist())
    assert oracle.gemm_exact(xq, wq).tolist() == exp
    assert oracle.gemm_int64_rows(xq, wq).tolist() == exp


def test_gemm_one_hot_and_bound():
    rng = np.random.default_rng(5)
    wq = rng.integers(-127, 128, (10, 20)).astype(np.int8)
    eye = np.eye(20, dtype=np.int8)
    # one-hot rows pick out the columns of wq
    assert np.array_equal(oracle.gemm_exact(eye, wq), wq.T.astype(np.int32))
    # the extreme +-127 products reach 127^2 K exactly at the largest K
    K = oracle.K_MAX
    assert K == 133144
    a = np.full((2, K), 127, np.int8)
    a[1] = -127
    b = np.full((1, K), 127, np.int8)
    acc = oracle.gemm_exact(a, b)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K
    assert acc[0, 0] <= 2**31 - 1
    with pytest.raises(ValueError):
        oracle.gemm_exact(np.zeros((1, K + 1), np.int8), np.zeros((1, K + 1), np.int8))


def test_gemm_invariants():
    rng = np.random.default_rng(6)
    xq = rng.integers(-127, 128, (13, 200)).astype(np.int8)
    wq = rng.integers(-127, 128, (30, 200)).astype(np.int8)
    acc = oracle.gemm_exact(xq, wq)
    # a permutation of K applied to both operands changes nothing
    p = rng.permutation(200)
    assert np.array_equal(oracle.gemm_exact(xq[:, p], wq[:, p]), acc)
    # concatenating weights along N (fused QKV) equals separate products
    parts = [oracle.gemm_exact(xq, wq[a:b]) for a, b in ((0, 7), (7, 19), (19, 30))]
    assert np.array_equal(np.concatenate(parts, axis=1), acc)
    # sampled int64 rows agree
    rows = [0, 6, 12]
    assert np.array_equal(oracle.gemm_int64_rows(xq, wq, rows), acc[rows])


@pytest.mark.parametrize("case", epilogue_cases())
def test_epilogue_hand_cases(case):
    acc, sa, sw, bias, y = case
    b = None if bias is None else np.array([bias], np.uint16)
    got = oracle.epilogue(np.array([[acc]], np.int32), np.array([sa], np.float32),
                          np.array([sw], np.float32), b)
    assert int(got[0, 0]) == y


def test_epilogue_exact_rational_random():
    """fp32 steps and the bf16 cast against exact rationals (no FMA)."""
    rng = np.random.default_rng(7)
    acc = rng.integers(-(2**30), 2**30, (6, 9)).astype(np.int32)
    acc[0, :3] = [16777217, -16777219, 2**31 - 1]     # int -> fp32 rounding
    s_a = (rng.uniform(1e-4, 1e-1, 6)).astype(np.float32)
    s_w = (rng.uniform(1e-5, 1e-3, 9)).astype(np.float32)
    bias = to_bf16_bits(rng.normal(0.0, 0.01, 9))
    t = oracle.epilogue_f32(acc, s_a, s_w, bias)
    y = oracle.epilogue(acc, s_a, s_w, bias)
    bf = oracle.bf16_bits_to_f32(bias)
    for m in range(6):
        for n in range(9):
            e = to_f32(Fraction(int(acc[m, n])))
            e = f32_mul(float(e), float(s_a[m]))
            e = f32_mul(float(e), float(s_w[n]))
            e = f32_add(float(e), float(bf[n]))
            assert Fraction(float(t[m, n])) == e
            assert int(y[m, n]) == exact_bf16(e)


def test_bf16_rounding_matches_torch():
    """The oracle's bit-level RNE cast equals torch-CPU's float -> bfloat16."""
    rng = np.random.default_rng(8)
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and values near the overflow threshold
    ties = (rng.integers(0, 2**16, 5000).astype(np.uint32) << 16) | np.uint32(0x8000)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x00008000, 0x00018000,
                     0x80008000], np.uint32)
    u = np.concatenate([u, ties, edge])
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_epilogue_bias_optional_and_zero_acc():
    s_a = np.array([0.5, 0.0], np.float32)
    s_w = np.array([2.0, 4.0, 8.0], np.float32)
    acc = np.zeros((2, 3), np.int32)
    bias = np.array([0x3F80, 0xC000, 0x0000], np.uint16)   # 1, -2, 0
    assert oracle.epilogue(acc, s_a, s_w, bias).tolist() == [[0x3F80, 0xC000, 0]] * 2
    assert np.all(oracle.epilogue(acc, s_a, s_w, None) == 0)
