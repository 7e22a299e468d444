"""The C ABI of libw8a8 on the CPU: the library loads, exports every symbol
include/w8a8.h declares, and rejects invalid arguments before launching
anything (no GPU needed: every call here returns during validation)."""
import ctypes
import os
import re

import pytest

import w8a8_int8_dynamic_quant_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

P = ctypes.c_void_p
A = 0x10000          # a fake, 256-byte aligned device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(w8a(?:8|16)_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_symbols():
    assert header_functions() == sorted(w8.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = w8.lib()
    for name in header_functions():
        assert hasattr(L, name), name


def test_constants_match_header():
    text = open(HEADER).read()
    assert f"#define W8A8_K_MAX {w8.K_MAX}" in text
    assert f"#define W8A8_SMALL_M {w8.SMALL_M}" in text
    assert f"#define W8A8_SMALL_M_WIDE {w8.SMALL_M_WIDE}" in text
    assert "#define W8A8_LDO_MAX (1 << 22)" in text and w8.LDO_MAX == 1 << 22
    assert w8.K_MAX == (2**31 - 1) // (127 * 127)


def q(fn, *args):
    return getattr(w8.lib(), fn)(*args)


@pytest.mark.parametrize("fn", ["w8a8_quant_act", "w8a8_quantize_weights",
                                "w8a8_quant_act_f16", "w8a8_quantize_weights_f16"])
def test_quant_validation(fn):
    ok = (P(A), 4, 64, 64, P(A), P(A), None)
    assert q(fn, P(A), -1, 64, 64, P(A), P(A), None) == w8.ERR_INVALID_ARG
    for K in (0, 8, 24, 100, w8.K_MAX + 16):
        assert q(fn, P(A), 4, K, 4096 * 64, P(A), P(A), None) == w8.ERR_UNSUPPORTED, K
    assert q(fn, P(A), 4, -16, 64, P(A), P(A), None) == w8.ERR_INVALID_ARG
    assert q(fn, P(A), 4, 64, 48, P(A), P(A), None) == w8.ERR_INVALID_ARG      # ld < K
    assert q(fn, P(A), 4, 64, 68, P(A), P(A), None) == w8.ERR_UNSUPPORTED      # ld % 8
    assert q(fn, None, 4, 64, 64, P(A), P(A), None) == w8.ERR_INVALID_ARG
    assert q(fn, P(A), 4, 64, 64, None, P(A), None) == w8.ERR_INVALID_ARG
    assert q(fn, P(A), 4, 64, 64, P(A), None, None) == w8.ERR_INVALID_ARG
    assert q(fn, P(A + 2), 4, 64, 64, P(A), P(A), None) == w8.ERR_MISALIGNED
    assert q(fn, P(A), 4, 64, 64, P(A + 8), P(A), None) == w8.ERR_MISALIGNED
    assert q(fn, P(A), 4, 64, 64, P(A), P(A + 2), None) == w8.ERR_MISALIGNED
    # M == 0 is a no-op, even with NULL buffers
    assert q(fn, None, 0, 64, 64, None, None, None) == w8.OK
    assert ok  # the valid call itself would launch; it is exercised on the GPU


@pytest.mark.parametrize("f", ["w8a8_scaled_mm", "w8a8_scaled_mm_f16"])
def test_scaled_mm_validation(f):
    base = [P(A), P(A), 4, 64, P(A), P(A), 8, None, P(A), 8, None, None]

    def call(**kw):
        a = list(base)
        names = ["xq", "sa", "M", "K", "wq", "sw", "N", "bias", "out", "ldo", "acc", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(M=-1) == w8.ERR_INVALID_ARG
    assert call(N=0) == w8.ERR_INVALID_ARG
    assert call(K=40) == w8.ERR_UNSUPPORTED
    assert call(K=w8.K_MAX + 16) == w8.ERR_UNSUPPORTED
    assert call(ldo=7) == w8.ERR_INVALID_ARG
    assert call(xq=None) == w8.ERR_INVALID_ARG
    assert call(wq=None) == w8.ERR_INVALID_ARG
    assert call(out=None) == w8.ERR_INVALID_ARG
    assert call(sw=None) == w8.ERR_INVALID_ARG
    assert call(sa=None) == w8.ERR_INVALID_ARG
    assert call(xq=P(A + 4)) == w8.ERR_MISALIGNED
    assert call(wq=P(A + 4)) == w8.ERR_MISALIGNED
    assert call(sw=P(A + 2)) == w8.ERR_MISALIGNED
    assert call(bias=P(A + 1)) == w8.ERR_MISALIGNED
    assert call(acc=P(A + 2)) == w8.ERR_MISALIGNED
    assert call(M=0, xq=None, sa=None, wq=None, sw=None, out=None) == w8.OK
    # 32-bit tile addressing: ldo and, with debug accumulators, N are bounded
    assert call(ldo=w8.LDO_MAX + 1) == w8.ERR_UNSUPPORTED
    assert call(ldo=w8.LDO_MAX, acc=None, xq=None) == w8.ERR_INVALID_ARG   # ldo itself is fine
    big = w8.LDO_MAX // 2 + 1
    assert call(N=big, ldo=big, acc=P(A)) == w8.ERR_UNSUPPORTED


@pytest.mark.parametrize("f", ["w8a8_linear", "w8a8_linear_f16"])
def test_linear_validation(f):
    M, K, N = 32, 64, 8
    ws = w8.workspace_bytes(M, K, N)
    base = [P(A), M, K, K, P(A), P(A), N, None, P(A), N, P(A), ws, None, None]
    names = ["x", "M", "K", "ldx", "wq", "sw", "N", "bias", "out", "ldo", "ws", "wsb", "acc", "st"]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(M=-3) == w8.ERR_INVALID_ARG
    assert call(K=0) == w8.ERR_UNSUPPORTED
    assert call(ldx=32) == w8.ERR_INVALID_ARG
    assert call(ldx=68) == w8.ERR_UNSUPPORTED
    assert call(x=None) == w8.ERR_INVALID_ARG
    assert call(x=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(ws=None) == w8.ERR_WORKSPACE
    assert call(wsb=ws - 1) == w8.ERR_WORKSPACE
    assert call(ws=P(A + 4)) == w8.ERR_MISALIGNED
    assert call(M=0, x=None, ws=None, wsb=0) == w8.OK


def test_workspace_and_path_queries():
    assert w8.workspace_bytes(0, 64, 8) == 0
    assert w8.workspace_bytes(1, 64, 8) == 256 + 256
    assert w8.workspace_bytes(4352, 3072, 9216) == 4352 * 3072 + 17408
    assert w8.linear_path(0, 64, 8) == w8.PATH_NONE
    for m in (1, 2, 8, 16, 17, 32):
        assert w8.linear_path(m, 3072, 18432) == w8.PATH_SMALL_M
    for m in (33, 4352):
        assert w8.linear_path(m, 3072, 18432) == w8.PATH_GEMM
    # the small-M kernel keeps the quantised rows in LDS: longer rows use the GEMM
    assert w8.linear_path(16, 8192, 64) == w8.PATH_SMALL_M
    assert w8.linear_path(1, 8208, 64) == w8.PATH_GEMM
    assert w8.linear_path(32, 4096, 64) == w8.PATH_SMALL_M
    assert w8.linear_path(17, 4112, 64) == w8.PATH_GEMM
    assert w8.linear_path(4, 20, 8) == w8.ERR_UNSUPPORTED
    assert w8.linear_path(-1, 64, 8) == w8.ERR_INVALID_ARG
    bm, bn = w8.gemm_tile(4352, 3072, 9216)
    assert bm >= 128 and bn >= 128
    # 65..127 rows: 128x128 tiles when two K pieces of them fill 256 CUs
    assert w8.gemm_tile(64, 3072, 18432) == (64, 64)
    assert w8.gemm_tile(65, 3072, 32768) == (128, 128)
    assert w8.gemm_tile(127, 3072, 16256) == (64, 64)
    assert w8.gemm_tile(127, 3072, 16384) == (128, 128)
    # split K (on a device of 256 compute units, the count assumed without a
    # GPU): the workspace adds int32 partial sums after xq and a_scale, on
    # 128x128 and 64x64 tiles only (256x256 tiles that fill at most half of
    # the compute units run as 128-row halves instead, with no partial sums)
    base = lambda M, K: ((M * K + 255) // 256) * 256 + ((4 * M + 255) // 256) * 256
    assert w8.workspace_bytes(512, 4096, 12288) == base(512, 4096)      # 96 256x256 tiles
    assert w8.workspace_bytes(700, 2000, 8200) == base(700, 2000)       # 99 256x256 tiles
    assert w8.workspace_bytes(512, 4096, 4096) == base(512, 4096) + 2 * 512 * 4096 * 4  # 128 tiles
    assert w8.workspace_bytes(1024, 4096, 4096) == base(1024, 4096) + 2 * 1024 * 4096 * 4
    assert w8.workspace_bytes(1024, 4096, 4104) == base(1024, 4096)     # 68 256x256 tiles
    assert w8.workspace_bytes(256, 3072, 18432) == base(256, 3072)      # 288 128x128 tiles
    assert w8.workspace_bytes(64, 3072, 18432) == base(64, 3072) + 3 * 64 * 18432 * 4
    assert w8.workspace_bytes(64, 4096, 4096) == base(64, 4096) + 4 * 64 * 4096 * 4
    assert w8.workspace_bytes(100, 3072, 18432) == base(100, 3072) + 2 * 100 * 18432 * 4  # 128
    assert w8.workspace_bytes(100, 3072, 40000) == base(100, 3072)      # 313 128x128 tiles
    assert w8.workspace_bytes(40, 960, 1024) == base(40, 960)           # K too short
    assert w8.workspace_bytes(32, 3072, 18432) == base(32, 3072)        # small-M path
    assert w8.workspace_bytes(4352, 3072, 9216) == base(4352, 3072)      # enough tiles
    assert w8.workspace_bytes(512, 4096, 12296) == base(512, 4096)      # 98 256x256 tiles
    assert w8.workspace_bytes(512, 4096, 12292) == base(512, 4096)       # N % 8 != 0
    assert w8.workspace_bytes(512, 768, 12288) == base(512, 768)         # K too short


def test_unpack_validation():
    f = "w8a8_unpack_pack_quantized"
    base = [P(A), 8, 64, 16, P(A), w8.SCALE_F32, P(A), P(A), None]
    names = ["packed", "N", "K", "ldp", "scale", "dtype", "wq", "ws", "st"]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(N=-1) == w8.ERR_INVALID_ARG
    assert call(K=40) == w8.ERR_UNSUPPORTED
    assert call(K=0) == w8.ERR_UNSUPPORTED
    assert call(ldp=15) == w8.ERR_INVALID_ARG            # ldp < K/4
    assert call(ldp=18) == w8.ERR_UNSUPPORTED            # ldp % 4
    assert call(dtype=3) == w8.ERR_INVALID_ARG
    assert call(packed=None) == w8.ERR_INVALID_ARG
    assert call(scale=None) == w8.ERR_INVALID_ARG
    assert call(wq=None) == w8.ERR_INVALID_ARG
    assert call(ws=None) == w8.ERR_INVALID_ARG
    assert call(packed=P(A + 4)) == w8.ERR_MISALIGNED
    assert call(wq=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(ws=P(A + 2)) == w8.ERR_MISALIGNED
    assert call(scale=P(A + 2)) == w8.ERR_MISALIGNED     # fp32 scales need 4 bytes
    assert call(N=0, packed=None, scale=None, wq=None, ws=None) == w8.OK
    assert f"#define W8A8_SCALE_BF16 {w8.SCALE_BF16}" in open(HEADER).read()
    # weights that may hold -128: 127 * 128 * K must stay below 2^31
    assert f"#define W8A8_K_MAX_PACKED {w8.K_MAX_PACKED}" in open(HEADER).read()
    assert 127 * 128 * w8.K_MAX_PACKED < 2**31 <= 127 * 128 * (w8.K_MAX_PACKED + 1)
    for K in (132112, w8.K_MAX - w8.K_MAX % 16):
        assert call(K=K, ldp=K // 4 + (-(K // 4)) % 4) == w8.ERR_UNSUPPORTED, K


def test_w8a16_validation():
    f = "w8a16_linear"
    base = [P(A), 4, 3072, 3072, P(A), P(A), 64, None, P(A), 64, None]
    names = ["x", "M", "K", "ldx", "wq", "sw", "N", "bias", "out", "ldo", "st"]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(M=-1) == w8.ERR_INVALID_ARG
    assert call(M=17) == w8.ERR_UNSUPPORTED                   # small-M path only
    assert call(M=16, K=3984, ldx=3984) == w8.ERR_UNSUPPORTED   # activations exceed LDS
    assert call(M=8, K=8080, ldx=8080) == w8.ERR_UNSUPPORTED
    assert call(K=40, ldx=40) == w8.ERR_UNSUPPORTED
    assert call(ldx=3000) == w8.ERR_INVALID_ARG
    assert call(ldx=3076) == w8.ERR_UNSUPPORTED
    assert call(x=None) == w8.ERR_INVALID_ARG
    assert call(wq=None) == w8.ERR_INVALID_ARG
    assert call(x=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(bias=P(A + 1)) == w8.ERR_MISALIGNED
    assert call(M=0, x=None) == w8.OK
    assert f"#define W8A16_MAX_M {w8.W8A16_MAX_M}" in open(HEADER).read()


def test_layernorm_modulate_validation():
    f = "w8a8_layernorm_modulate_quant_act"
    names = ["x", "M", "K", "ldx", "sh", "sc", "ldm", "rpg", "eps", "xq", "sa", "y", "ldy", "st"]
    base = [P(A), 4, 3072, 3072, P(A), P(A), 3072, 4, ctypes.c_float(1e-6), P(A), P(A), None, 0,
            None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = ctypes.c_float(v) if k == "eps" else v
        return q(f, *a)

    assert call(M=-1) == w8.ERR_INVALID_ARG
    assert call(K=16400, ldx=16400, ldm=16400) == w8.ERR_UNSUPPORTED    # past the LN limit
    assert call(K=40, ldx=40, ldm=40) == w8.ERR_UNSUPPORTED
    assert call(ldx=3000) == w8.ERR_INVALID_ARG
    assert call(ldx=3076) == w8.ERR_UNSUPPORTED
    assert call(ldm=3064) == w8.ERR_INVALID_ARG
    assert call(ldm=3076) == w8.ERR_UNSUPPORTED
    assert call(rpg=0) == w8.ERR_INVALID_ARG
    for eps in (0.0, -1e-6, float("inf"), float("nan")):
        assert call(eps=eps) == w8.ERR_INVALID_ARG, eps
    assert call(y=P(A), ldy=3000) == w8.ERR_INVALID_ARG
    assert call(y=P(A), ldy=3076) == w8.ERR_UNSUPPORTED
    for k in ("x", "sh", "sc", "xq", "sa"):
        assert call(**{k: None}) == w8.ERR_INVALID_ARG, k
    for k in ("x", "sh", "sc", "xq", "y"):
        kw = {k: P(A + 8)}
        if k == "y":
            kw["ldy"] = 3072
        assert call(**kw) == w8.ERR_MISALIGNED, k
    assert call(sa=P(A + 2)) == w8.ERR_MISALIGNED
    assert call(M=0, x=None, sh=None, sc=None, xq=None, sa=None) == w8.OK
    assert w8.PRODUCER_MAX_K["layernorm"] == 16384


def test_gelu_validation():
    f = "w8a8_gelu_quant_act"
    names = ["z", "M", "K", "ldz", "approx", "xq", "sa", "y", "ldy", "st"]
    base = [P(A), 4, 12288, 12288, 0, P(A), P(A), None, 0, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(approx=2) == w8.ERR_INVALID_ARG
    assert call(approx=-1) == w8.ERR_INVALID_ARG
    assert call(M=-1) == w8.ERR_INVALID_ARG
    assert call(K=32784, ldz=32784) == w8.ERR_UNSUPPORTED
    assert call(K=24, ldz=24) == w8.ERR_UNSUPPORTED
    assert call(ldz=12280) == w8.ERR_INVALID_ARG
    assert call(ldz=12292) == w8.ERR_UNSUPPORTED
    assert call(y=P(A), ldy=12280) == w8.ERR_INVALID_ARG
    for k in ("z", "xq", "sa"):
        assert call(**{k: None}) == w8.ERR_INVALID_ARG, k
    assert call(z=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(xq=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(y=P(A + 8), ldy=12288) == w8.ERR_MISALIGNED
    assert call(M=0, z=None, xq=None, sa=None) == w8.OK
    text = open(HEADER).read()
    assert f"#define W8A8_GELU_ERF {w8.GELU_ERF}" in text
    assert f"#define W8A8_GELU_TANH {w8.GELU_TANH}" in text
    assert w8.PRODUCER_MAX_K["gelu"] == 32768


def test_linear_noalloc_validation():
    """Arguments are checked as w8a8_linear checks them, and shapes whose
    workspace would exceed the library's scratch array are refused, all
    before anything touches a device."""
    f = "w8a8_linear_noalloc"
    base = [P(A), 8, 64, 64, P(A), P(A), 16, None, P(A), 16, None, None]
    names = ["x", "M", "K", "ldx", "wq", "ws", "N", "bias", "out", "ldo", "acc", "st"]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(f, *a)

    assert call(M=-1) == w8.ERR_INVALID_ARG
    assert call(N=0) == w8.ERR_INVALID_ARG
    assert call(K=40, ldx=40) == w8.ERR_UNSUPPORTED
    assert call(ldx=48) == w8.ERR_INVALID_ARG
    assert call(ldo=8) == w8.ERR_INVALID_ARG
    assert call(x=None) == w8.ERR_INVALID_ARG
    assert call(wq=None) == w8.ERR_INVALID_ARG
    assert call(out=None) == w8.ERR_INVALID_ARG
    assert call(x=P(A + 8)) == w8.ERR_MISALIGNED
    assert call(M=0, x=None, wq=None, ws=None, out=None) == w8.OK
    assert f"#define W8A8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in open(HEADER).read()
    # the largest DiT block activation (4352 x 12288) fits; 8192 x 8192 does not
    assert w8.workspace_bytes(4352, 12288, 3072) <= w8.NOALLOC_SCRATCH_BYTES
    assert w8.workspace_bytes(8192, 8192, 64) > w8.NOALLOC_SCRATCH_BYTES
    assert call(M=8192, K=8192, ldx=8192, N=64, ldo=64) == w8.ERR_WORKSPACE


def test_launch_failure_reports_hip_error():
    """A call that passes validation but whose launch fails returns
    W8A8_ERR_HIP and records the hipError_t for w8a8_last_hip_error (here
    the launch fails because no device is visible); the caller can then fall
    back with the logged reason (unsloth test_diffusion_transformer_quant.py
    commit log: a quantisation failure falls back, with the reason logged)."""
    import subprocess
    import sys
    code = (
        "import ctypes, sys\n"
        "L = ctypes.CDLL(sys.argv[1])\n"
        "P, I = ctypes.c_void_p, ctypes.c_int64\n"
        "L.w8a8_quant_act.argtypes = [P, I, I, I, P, P, P]\n"
        "L.w8a8_linear.argtypes = [P, I, I, I, P, P, I, P, P, I, P, ctypes.c_size_t, P, P]\n"
        "L.w8a8_linear_workspace_bytes.restype = ctypes.c_size_t\n"
        "L.w8a8_linear_workspace_bytes.argtypes = [I, I, I]\n"
        "a = 0x10000\n"
        "s1 = L.w8a8_quant_act(a, 4, 64, 64, a, a, None)\n"
        "e1 = L.w8a8_last_hip_error()\n"
        "ws = L.w8a8_linear_workspace_bytes(64, 256, 128)\n"
        "s2 = L.w8a8_linear(a, 64, 256, 256, a, a, 128, None, a, 128, a, ws, None, None)\n"
        "print(s1, e1, s2, L.w8a8_last_hip_error())\n")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code, w8.LIB_PATH], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    s1, e1, s2, e2 = map(int, r.stdout.split()[-4:])
    assert (s1, s2) == (w8.ERR_HIP, w8.ERR_HIP)
    assert e1 != 0 and e2 != 0
    assert w8.status_string(s1) == "HIP launch failed"


def test_status_strings():
    for s in (w8.OK, w8.ERR_INVALID_ARG, w8.ERR_UNSUPPORTED, w8.ERR_MISALIGNED,
              w8.ERR_WORKSPACE, w8.ERR_HIP):
        assert w8.status_string(s) and w8.status_string(s) != "unknown status"
    assert w8.status_string(12345) == "unknown status"
    assert q("w8a8_last_hip_error") == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        w8.quant_act(torch.zeros((2, 16), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        w8.quant_act(torch.zeros((2, 16), dtype=torch.float32))
    with pytest.raises(ValueError):
        w8.quant_act(torch.zeros((2, 16), dtype=torch.float16))
    with pytest.raises(TypeError):
        w8.quantize_weights(torch.zeros((2, 16), dtype=torch.float64))
