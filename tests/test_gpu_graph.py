"""w8a8_linear and the fused GELU producer captured in a HIP graph
(torch.cuda.graph) and replayed.

Every path (the small-M kernel, quantisation + GEMM, 256x256 tiles run as
halves, K split on 128x128 and 64x64 tiles with its reduction kernel)
launches only kernels on the caller's stream,
with no allocation, copy or memset, so a graph holds the whole linear. Each
replay follows new activations copied into the captured input and is compared
bit for bit with an eager call on the same activations, with eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

import w8a8_int8_dynamic_quant_amd as w8
from gpu_util import announce, dev_bf16, host_bits
from synth_inputs import random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K,with_bias", [
    (1, 18432, 3072, True),      # small-M row modes, one row per wave
    (12, 200, 3072, True),       # small-M split kernel, rows staged in LDS
    (32, 4096, 4096, False),     # small-M split kernel, four token blocks, rows read twice
    (1, 8192, 4096, True),       # small-M split kernel, two weight waves per row group
    (300, 700, 1296, True),      # quantisation + GEMM, one pass
    (64, 4096, 4096, True),      # 64x64 tiles, K split in four
    (512, 4096, 4096, False),    # 128x128 tiles, K split in two
    (512, 12288, 4096, True),    # 256x256 tiles, every tile as two 128-row halves
])
def test_linear_graph_replays(M, N, K, with_bias):
    rng = np.random.default_rng(M * 7 + N + K)
    wq, sw = w8.quantize_weights(dev_bf16(random_bf16(rng, (N, K), 0.02)))
    b = dev_bf16(random_bf16(rng, (N,), 0.01)) if with_bias else None
    x = dev_bf16(random_bf16(rng, (M, K)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((max(w8.workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device="cuda")
    announce(f"graph capture of w8a8_linear M={M} N={N} K={K} bias={with_bias} "
             f"path={w8.linear_path(M, K, N)} workspace={ws.numel()}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w8.linear(x, wq, sw, b, out=y, workspace=ws)      # warm-up off the default stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.linear(x, wq, sw, b, out=y, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        xs = dev_bf16(random_bf16(rng, (M, K)))
        x.copy_(xs)
        torch.cuda.synchronize()
        announce(f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = host_bits(y).copy()
        ref = w8.linear(xs, wq, sw, b)      # eager, with its own output and workspace
        torch.cuda.synchronize()
        assert np.array_equal(got, host_bits(ref)), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("approximate", ["none", "tanh"])
def test_gelu_quant_graph_replays(approximate):
    """The fused GELU + quantisation on its table path (M*K >= 2^22): the
    table kernel and the quantising kernel replay from the graph."""
    M, K = 1400, 3072
    rng = np.random.default_rng(17 if approximate == "none" else 18)
    z = dev_bf16(random_bf16(rng, (M, K)))
    announce(f"graph capture of w8a8_gelu_quant_act {approximate} M={M} K={K}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w8.gelu_quant_act(z, approximate, return_y=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = w8.gelu_quant_act(z, approximate, return_y=True)
    torch.cuda.synchronize()
    for rep in range(3):
        zs = dev_bf16(random_bf16(rng, (M, K)))
        z.copy_(zs)
        torch.cuda.synchronize()
        announce(f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = [o.detach().cpu().clone() for o in outs]
        ref = w8.gelu_quant_act(zs, approximate, return_y=True)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               (b.view(torch.int16) if b.dtype == torch.bfloat16 else b).cpu()), \
                f"replay {rep} differs from the eager call"
