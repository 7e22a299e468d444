"""w8a8_linear_noalloc (the workspace comes from the library's per-GPU
scratch array, for callers that cannot allocate) against w8a8_linear through
the C ABI: the same kernels, so the same int32 accumulators and the same
output bits, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), across the small-M path, the
one-pass GEMM and the K split whose partial sums live in the scratch."""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, assert_bf16_close, assert_equal, dev_bf16, host, host_bits
from synth_inputs import random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _run_pair(M, K, N, with_bias, seed):
    rng = np.random.default_rng(seed)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    b = random_bf16(rng, (N,), 0.01) if with_bias else None
    wq, sw = w8.quantize_weights(dev_bf16(w))
    xd = dev_bf16(x)
    bd = None if b is None else dev_bf16(b)
    acc_ref = torch.empty((M, N), dtype=torch.int32, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    announce(f"noalloc M={M} K={K} N={N} bias={with_bias} "
             f"path={w8.linear_path(M, K, N)} workspace={w8.workspace_bytes(M, K, N)}")
    y_ref = w8.linear(xd, wq, sw, bd, acc_debug=acc_ref)
    y = w8.linear_noalloc(xd, wq, sw, bd, out=out, acc_debug=acc)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert_equal(host(acc), host(acc_ref), "acc")
    assert_equal(host_bits(y), host_bits(y_ref), "y")
    # and to the oracle's bar
    wq_e, sw_e = oracle.quantize_weights(w)
    exp = oracle.linear(x, wq_e, sw_e, b)
    assert_equal(host(acc), exp["acc"], "acc vs oracle")
    assert_bf16_close(host_bits(y), exp["y"])


@pytest.mark.parametrize("first,second", [
    # K split in two on 128x128 tiles (partial sums in the scratch), then a one-pass GEMM
    ((512, 4096, 4096, True), (300, 1040, 700, False)),
    # one-pass GEMM, then the fused small-M kernel
    ((1024, 3072, 3072, False), (8, 3072, 1024, True)),
    # the small-M split kernel (rows staged in LDS), then its row-mode kernel
    ((16, 3072, 4096, True), (1, 1040, 520, True)),
])
def test_noalloc_matches_linear_on_two_calls(first, second):
    _run_pair(*first, seed=1)
    _run_pair(*second, seed=2)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    x = torch.zeros((8192, 8192), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((64, 8192), dtype=torch.int8, device="cuda")
    sw = torch.ones((64,), dtype=torch.float32, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:
        w8.linear_noalloc(x, wq, sw)
    assert e.value.status == w8.ERR_WORKSPACE
