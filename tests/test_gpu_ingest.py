"""GPU parity of the compressed-tensors pack-quantized ingest
(w8a8_unpack_pack_quantized) against the oracle: bit-exact int8 weights and
fp32 scales, for every scale type, padded rows, and the DiT weight sizes; and
the unpacked weights drive the linear exactly like quantised ones."""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, assert_bf16_close, assert_equal, dev, dev_bf16, host, host_bits
from synth_inputs import random_bf16, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _words(rng, N, W):
    return rng.integers(-(1 << 31), 1 << 31, size=(N, W), dtype=np.int64).astype(np.int32)


def _scales(rng, N, kind):
    v = rng.uniform(1e-4, 1e-2, N)
    if kind == "f32":
        return v.astype(np.float32), torch.from_numpy(v.astype(np.float32))
    if kind == "bf16":
        bits = to_bf16_bits(v)
        return bits, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    bits = v.astype(np.float16).view(np.uint16)
    return bits, torch.from_numpy(bits.view(np.int16)).view(torch.float16)


@pytest.mark.parametrize("N,K,ldp", [(1, 16, 4), (7, 48, 16), (33, 1040, 264), (300, 3072, 768),
                                     (9216, 3072, 768), (3072, 12288, 3072)])
@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
def test_unpack_parity(N, K, ldp, kind):
    rng = np.random.default_rng(N + K + ldp)
    words = _words(rng, N, ldp)
    sc_host, sc_t = _scales(rng, N, kind)
    announce(f"unpack N={N} K={K} ldp={ldp} scale={kind}")
    wq, s = w8.unpack_pack_quantized(dev(words)[:, : K // 4] if ldp != K // 4 else dev(words),
                                     sc_t.reshape(N, 1).cuda())
    torch.cuda.synchronize()
    assert_equal(host(wq), oracle.unpack_pack_quantized(words[:, : K // 4]), "wq")
    assert_equal(host(s), oracle.scale_to_f32(sc_host, kind), "w_scale")


def test_unpacked_weights_drive_the_linear():
    """Pack the oracle's quantised weights, unpack on the GPU, run the linear:
    the same int32 accumulators and outputs as the oracle's layer."""
    rng = np.random.default_rng(17)
    M, K, N = 70, 512, 320
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    wq_e, sw_e = oracle.quantize_weights(w)
    u = (wq_e.astype(np.int64) + 128) & 0xFF
    words = sum(u[:, j::4] << (8 * j) for j in range(4))
    words = np.where(words >= 1 << 31, words - (1 << 32), words).astype(np.int32)
    announce("unpack -> linear")
    wq, sw = w8.unpack_pack_quantized(dev(words), torch.from_numpy(sw_e).cuda())
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = w8.linear(dev_bf16(x), wq, sw, None, acc_debug=acc)
    torch.cuda.synchronize()
    exp = oracle.linear(x, wq_e, sw_e, None)
    assert_equal(host(acc), exp["acc"], "acc")
    assert_bf16_close(host_bits(y), exp["y"])
