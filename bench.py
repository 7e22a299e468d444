"""Benchmark of the W8A8 int8-dynamic linear on one MI355X.

One step = one pass of the whole hot path over one 1024px diffusion
transformer block: the four block linears at M = 4352 tokens (fused QKV
3072->9216, out-proj 3072->3072, FFN up 3072->12288, FFN down 12288->3072),
each as dynamic activation quantisation + int8 MFMA GEMM with the fused
scale epilogue, plus the AdaLN modulation projection 3072->18432 at M = 1 on
the fused small-M kernel. Weights are quantised once before timing (load
time); inputs are synthetic (seeded, see synth_inputs) and resident in HBM.

Prints one JSON line. `value` is int8 TOPS of the whole step (wall clock
over the timed steps); per-shape figures, the roofline of the dominant kernel
(the GEMM, bound by int8 MFMA throughput) and the CPU oracle's rate on the
same step ride along. Inside the timed region HIP events, recorded with a
device-scope release (hipEventReleaseToDevice), bracket only the GEMM
launches; the full per-launch breakdown comes from a separate pass after it,
then a 2.5 s clock pass reads the graphics clock and socket power the chip
sustains on the step (`sclk`).

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--no-cpu-baseline]
                    [--no-next-rows]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("int8 TOPS + % of MI355X int8 MFMA peak (HBM GB/s for M≤16), per shape")
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
GEMM_KERNEL = "gemm_pp_kernel"          # the 256x256-tile kernel all four DiT shapes take
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_pp_dit_block_counters.json")


class HipEvents:
    """Timing events of the HIP runtime that torch and libw8a8 share (one
    runtime per process: both resolve libamdhip64.so.7 to torch's copy),
    created with hipEventReleaseToDevice: recording one releases at device
    scope only, so it does not write the caches back to memory the way a
    default (system-scope) event does, and the kernels between two events are
    timed without that cost."""
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        ev = ctypes.c_void_p()
        if self.h.hipEventCreateWithFlags(ctypes.byref(ev), self.RELEASE_TO_DEVICE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(ev)
        return ev

    def record(self, ev, stream) -> None:
        if self.h.hipEventRecord(ev, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        t = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def close(self) -> None:
        for ev in self.made:
            self.h.hipEventDestroy(ev)
        self.made.clear()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (profiling runs)")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the W8A16 / ingest / fp16 measurements after the block step")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), the "
                        "reference for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes")
    p.add_argument("--profile-linear", default="", metavar="M,K,N",
                   help="only run w8a8_linear (bias, bf16) on one shape, --steps calls after "
                        "--warmup, weights rotated over copies of 512 MB or more; for "
                        "rocprofv3 runs of a single shape")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.ones((n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def profile_linear(shape: str, steps: int, warmup: int) -> None:
    import torch

    import w8a8_int8_dynamic_quant_amd as w8
    M, K, N = (int(v) for v in shape.split(","))
    copies = max(2, -(-(512 << 20) // (N * K)))
    g = torch.Generator(device="cpu").manual_seed(11)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16).cuda()
    w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16).cuda()
    wq, sw = w8.quantize_weights(w)
    wqs = [wq.clone() for _ in range(copies)]
    bias = (torch.randn((N,), generator=g) * 0.01).to(torch.bfloat16).cuda()
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((max(1, w8.workspace_bytes(M, K, N)),), dtype=torch.uint8, device="cuda")
    for i in range(warmup):
        w8.linear(x, wqs[i % copies], sw, bias, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        w8.linear(x, wqs[i % copies], sw, bias, out=out, workspace=ws)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / max(1, steps) * 1e6
    print(json.dumps({"profile_linear": [M, K, N], "path": w8.linear_path(M, K, N),
                      "calls": steps, "us_per_call_wall": us}), flush=True)


# The sources the GEMM kernel is compiled from (its file and the headers it
# includes); the committed HBM counters stay valid while these are unchanged.
GEMM_SOURCES = ("gemm_i8.hip", "w8a8_device.h", "w8a8_kernels.h")


def align256(n: int) -> int:
    return (n + 255) // 256 * 256


def kernel_source_hash() -> str:
    csrc = os.path.join(ROOT, "w8a8_int8_dynamic_quant_amd", "csrc")
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_counters():
    """The committed rocprofv3 summary of the GEMM on this step (HBM bytes and
    kernel-trace duration per launch), or {} when the kernel sources changed
    since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return {}
    if c.get("kernel_source_hash") != kernel_source_hash():
        return {}
    return c


def cpu_baseline(inputs, wq_host, min_seconds: float = 10.0):
    """The oracle, as it stands, on whole steps (all five linears), repeated
    until at least `min_seconds` of CPU work."""
    import numpy as np

    import oracle
    ops = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        for name, d in inputs.items():
            wq, sw = wq_host[name]
            oracle.linear(d["x"], wq, sw, d["bias"])
            ops += 2 * d["M"] * d["N"] * d["K"]
        steps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return {
        "value": ops / dt / 1e12,
        "unit": "TOPS",
        # the oracle's matrix products run on the BLAS threads; the rest of it
        # (quantisation, epilogue) is single-threaded numpy
        "cores": threads or 1,
        "blas_threads": threads,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{steps} whole step(s): the 4 DiT block linears at M=4352 and the M=1 "
                  "modulation projection (quantise, exact int GEMM, fp32 epilogue)",
        "seconds": dt,
        "numpy": np.__version__,
    }


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def clock_pass(step, torch, seconds: float = 2.5):
    """The graphics clock (per XCD, MHz) and socket power (W) the chip
    sustains on the block step: amdsmi's GPU metrics, read every 50 ms while
    the step runs back to back for `seconds`. The metrics table refreshes
    about once a second, so only readings taken after the first second count
    (and each distinct reading once). Percent of a published peak depends on
    this clock. Returns None when amdsmi cannot be used."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    readings, stop = [], threading.Event()

    def sample():
        t0 = time.perf_counter()
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            except Exception:
                return
            xcd = [v for v in (m.get("current_gfxclks") or [])
                   if isinstance(v, (int, float)) and 0 < v < 10000]
            p = m.get("current_socket_power")
            readings.append((time.perf_counter() - t0, tuple(xcd),
                             p if isinstance(p, (int, float)) else None))
            stop.wait(0.05)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    seen, clk, power = set(), [], []
    for t, xcd, p in readings:
        if t < 1.0 or not xcd or (xcd, p) in seen:
            continue
        seen.add((xcd, p))
        clk.append(sum(xcd) / len(xcd))
        if p is not None:
            power.append(p)
    if not clk:
        return None
    return {"mean_mhz": sum(clk) / len(clk), "min_mhz": min(clk), "max_mhz": max(clk),
            "per_xcd_mhz": list(xcd), "socket_power_w": sum(power) / len(power) if power else None,
            "readings": len(clk),
            "source": (f"amdsmi gpu metrics (current gfx clock averaged over XCDs) read while the "
                       f"block step ran back to back for {seconds} s after the timed region")}


def next_rows(w8, torch, np, dev, to_dev) -> dict:
    """The layers beyond the block step, measured after it on their own.

    fp16 activations/outputs: the whole linear in fp16 against bf16 on the
    DiT QKV shape and the modulation projection (M = 1, 16).
    Modulation projection 3072->18432 at M = 1, 8, 16 with bias: W8A16
    (bf16 activations, int8 weights) against the W8A8 small-M kernel, both
    HBM-bound (the weight is read once), reported as algorithmic GB/s =
    (2MK + NK + 4N + 2N + 2MN) / t. Pack-quantized ingest of the same weight
    (N*K/4 words in, N*K int8 + N fp32 out). The modulated LayerNorm and GELU
    fused with the quantisation (fused_producers). The whole linear on the
    workload table's other configurations (baseline_configs). Each figure is the median over 5
    batches of 60 back-to-back calls bracketed by HIP events, rotating over
    copies of the weight that together exceed the 256 MB last-level cache.
    """
    from synth_inputs import make_linear_inputs
    lib = w8.lib()
    sp = torch.cuda.current_stream(dev)
    d = make_linear_inputs("mod_m16_3072x18432")
    K, N = d["K"], d["N"]
    n_copies = 10
    wq0, sw = w8.quantize_weights(to_dev(d["w"]))
    wqs = [wq0] + [wq0.clone() for _ in range(n_copies - 1)]
    bias, x = to_dev(d["bias"]), to_dev(d["x"])
    bias16, x16 = bias.to(torch.float16), x.to(torch.float16)   # fp16 activations
    out = torch.empty((16, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((w8.workspace_bytes(16, K, N),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def timed(fn, calls=60, batches=5):
        for i in range(10):
            fn(i)
        per_call = []
        for _ in range(batches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(sp)
            for i in range(calls):
                fn(i)
            e1.record(sp)
            e1.synchronize()
            per_call.append(e0.elapsed_time(e1) / calls)
        return float(np.median(per_call)) * 1e3

    def ok(st):
        if st != 0:
            raise RuntimeError(f"libw8a8 status {st}")

    res = {"shape": f"Mx{K}x{N}, bias", "modulation": {}}
    for M in (1, 8, 16):
        alg = 2 * M * K + N * K + 4 * N + 2 * N + 2 * M * N
        us16 = timed(lambda i: ok(lib.w8a16_linear(
            x.data_ptr(), M, K, K, wqs[i % n_copies].data_ptr(), sw.data_ptr(), N,
            bias.data_ptr(), out.data_ptr(), N, sp.cuda_stream)))
        us16h = timed(lambda i: ok(lib.w8a16_linear_f16(
            x16.data_ptr(), M, K, K, wqs[i % n_copies].data_ptr(), sw.data_ptr(), N,
            bias16.data_ptr(), out.data_ptr(), N, sp.cuda_stream)))
        us8 = timed(lambda i: ok(lib.w8a8_linear(
            x.data_ptr(), M, K, K, wqs[i % n_copies].data_ptr(), sw.data_ptr(), N,
            bias.data_ptr(), out.data_ptr(), N, ws.data_ptr(), ws.numel(), None,
            sp.cuda_stream)))
        res["modulation"][f"M{M}"] = {
            "w8a16_us": us16, "w8a16_gbs": alg / (us16 * 1e-6) / 1e9,
            "w8a16_pct_hbm": 100 * alg / (us16 * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "w8a16_f16_us": us16h, "w8a16_f16_gbs": alg / (us16h * 1e-6) / 1e9,
            "w8a8_us": us8, "w8a8_gbs": alg / (us8 * 1e-6) / 1e9,
            "w8a8_pct_hbm": 100 * alg / (us8 * 1e-6) / 1e9 / PEAK_HBM_GBS}
    del wqs

    # fp16 activations/outputs: the whole linear (quantisation + product +
    # epilogue), fp16 against bf16 on the same shapes and values.
    def linear_pair(M, K, N, with_bias, seed):
        g = torch.Generator(device="cpu").manual_seed(seed)
        x32 = torch.randn((M, K), generator=g)
        w32 = torch.randn((N, K), generator=g) * 0.02
        b32 = torch.randn((N,), generator=g) * 0.01 if with_bias else None
        r = {}
        for tag, dt, fn in (("bf16", torch.bfloat16, lib.w8a8_linear),
                            ("f16", torch.float16, lib.w8a8_linear_f16)):
            xx = x32.to(dt).to(dev)
            wq_, sw_ = w8.quantize_weights(w32.to(dt).to(dev))
            bb = None if b32 is None else b32.to(dt).to(dev)
            oo = torch.empty((M, N), dtype=dt, device=dev)
            wsz = torch.empty((w8.workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            us = timed(lambda i: ok(fn(
                xx.data_ptr(), M, K, K, wq_.data_ptr(), sw_.data_ptr(), N,
                None if bb is None else bb.data_ptr(), oo.data_ptr(), N, wsz.data_ptr(),
                wsz.numel(), None, sp.cuda_stream)), calls=20 if M > 16 else 60)
            r[f"{tag}_us"] = us
            if M > 16:
                r[f"{tag}_tops"] = 2 * M * N * K / (us * 1e-6) / 1e12
            del xx, wq_, sw_, bb, oo, wsz
        return r

    res["f16_linear"] = {
        "note": "whole linear per call, same shapes and values in both types",
        "qkv_4352x3072x9216": linear_pair(4352, 3072, 9216, False, 1),
        "mod_m1_3072x18432": linear_pair(1, 3072, 18432, True, 2),
        "mod_m16_3072x18432": linear_pair(16, 3072, 18432, True, 3),
    }
    n_pk = 5
    packed0 = (wq0.to(torch.int16) + 128).to(torch.uint8).view(torch.int32)
    packs = [packed0] + [packed0.clone() for _ in range(n_pk - 1)]
    outs = [torch.empty_like(wq0) for _ in range(n_pk)]
    s_out = torch.empty_like(sw)
    torch.cuda.synchronize()
    us = timed(lambda i: ok(lib.w8a8_unpack_pack_quantized(
        packs[i % n_pk].data_ptr(), N, K, K // 4, sw.data_ptr(), w8.SCALE_F32,
        outs[i % n_pk].data_ptr(), s_out.data_ptr(), sp.cuda_stream)))
    alg = 2 * N * K + 8 * N
    res["unpack_pack_quantized"] = {"us": us, "gbs": alg / (us * 1e-6) / 1e9,
                                    "pct_hbm": 100 * alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    del packs, outs
    res["fused_producers"] = fused_producers(w8, torch, np, dev, timed, ok)
    res["baseline_configs"] = baseline_configs(w8, torch, dev, to_dev, timed, ok)
    return res


def baseline_configs(w8, torch, dev, to_dev, timed, ok) -> dict:
    """The whole linear (w8a8_linear) on the other configurations of the
    workload table: the probe shapes (64x256x128 with bias, 512x4096x4096
    with outlier channels, 512x4096x12288 Student-t with bias) and the
    modulation projection at M = 2, 17, 32 (all three on the fused small-M
    kernel). Weights rotate over copies totalling more than 512 MB; algorithmic
    bytes 2MK + NK + 4N (+ 2N bias) + 2MN."""
    from synth_inputs import make_linear_inputs
    lib = w8.lib()
    sp = torch.cuda.current_stream(dev)
    out = {}
    for name in ("c1_64x256x128", "c2_512x4096x4096_outliers", "c3_512x4096x12288_student_t",
                 "mod_m2_3072x18432", "mod_m17_3072x18432", "mod_m32_3072x18432"):
        d = make_linear_inputs(name)
        M, K, N = d["M"], d["K"], d["N"]
        wq0, sw = w8.quantize_weights(to_dev(d["w"]))
        copies = max(1, min(40, -(-(512 << 20) // (N * K))))
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        x = to_dev(d["x"])
        bias = None if d["bias"] is None else to_dev(d["bias"])
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((max(w8.workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        us = timed(lambda i: ok(lib.w8a8_linear(
            x.data_ptr(), M, K, K, wqs[i % copies].data_ptr(), sw.data_ptr(), N,
            None if bias is None else bias.data_ptr(), y.data_ptr(), N, ws.data_ptr(),
            ws.numel(), None, sp.cuda_stream)))
        alg = 2 * M * K + N * K + 4 * N + (2 * N if bias is not None else 0) + 2 * M * N
        ops = 2 * M * N * K
        out[name] = {"us": us, "tops": ops / (us * 1e-6) / 1e12,
                     "pct_int8_peak": 100 * ops / (us * 1e-6) / 1e12 / PEAK_INT8_TOPS,
                     "gbs": alg / (us * 1e-6) / 1e9,
                     "pct_hbm": 100 * alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "path": "small_m" if w8.linear_path(M, K, N) == w8.PATH_SMALL_M else "gemm",
                     "weight_copies": copies}
        del wqs, x, y, ws
        torch.cuda.synchronize()
    return out


def fused_producers(w8, torch, np, dev, timed, ok) -> dict:
    """The modulated LayerNorm on the DiT block's 4352 x 3072 input and GELU on
    its 4352 x 12288 FFN-down input, each fused with the int8 quantisation:
    algorithmic bytes 2MK (bf16 in) + MK (int8 out) + 4M (scales), plus 4K
    (shift, scale) for the LayerNorm; the optional bf16 y adds 2MK. Against
    the two-pass route it replaces: the quantisation kernel alone on a bf16
    row (what fusion saves, beside the producer's own bf16 write), and
    torch's bf16 producer ops followed by that quantisation (context only).
    Inputs and outputs rotate over copies totalling more than 512 MB."""
    lib = w8.lib()
    sp = torch.cuda.current_stream(dev)
    out = {}
    g = torch.Generator(device="cpu").manual_seed(7)
    for name, M, K in (("layernorm_modulate", 4352, 3072), ("gelu_tanh", 4352, 12288),
                       ("gelu_erf", 4352, 12288)):
        copies = max(2, -(-(512 << 20) // (2 * M * K)))
        x0 = torch.randn((M, K), generator=g).to(torch.bfloat16)
        xs = [x0.to(dev) for _ in range(copies)]
        xqs = [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(copies)]
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        shift = (torch.randn((K,), generator=g) * 0.5).to(torch.bfloat16).to(dev)
        scale = (torch.randn((K,), generator=g) * 0.5).to(torch.bfloat16).to(dev)
        torch.cuda.synchronize()
        if name == "layernorm_modulate":
            def fused(i, yp=None):
                ok(lib.w8a8_layernorm_modulate_quant_act(
                    xs[i % copies].data_ptr(), M, K, K, shift.data_ptr(), scale.data_ptr(), K, M,
                    1e-6, xqs[i % copies].data_ptr(), sa.data_ptr(), yp, K, sp.cuda_stream))

            def producer_torch(xx):
                h = torch.nn.functional.layer_norm(xx, (K,), eps=1e-6)
                return h * (1 + scale) + shift
            mod_bytes = 4 * K
        else:
            code = w8.GELU_TANH if name == "gelu_tanh" else w8.GELU_ERF
            approx = "tanh" if name == "gelu_tanh" else "none"

            def fused(i, yp=None):
                ok(lib.w8a8_gelu_quant_act(xs[i % copies].data_ptr(), M, K, K, code,
                                           xqs[i % copies].data_ptr(), sa.data_ptr(), yp, K,
                                           sp.cuda_stream))

            def producer_torch(xx):
                return torch.nn.functional.gelu(xx, approximate=approx)
            mod_bytes = 0
        alg = 3 * M * K + 4 * M + mod_bytes
        calls = 60 if K <= 4096 else 20
        us = timed(lambda i: fused(i), calls=calls)
        us_y = timed(lambda i: fused(i, y.data_ptr()), calls=calls)
        us_q = timed(lambda i: ok(lib.w8a8_quant_act(
            xs[i % copies].data_ptr(), M, K, K, xqs[i % copies].data_ptr(), sa.data_ptr(),
            sp.cuda_stream)), calls=calls)
        us_t = timed(lambda i: w8.quant_act(producer_torch(xs[i % copies])), calls=calls)
        out[name] = {
            "shape": f"{M}x{K}", "fused_us": us, "fused_gbs": alg / (us * 1e-6) / 1e9,
            "fused_pct_hbm": 100 * alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "fused_with_y_us": us_y, "quant_alone_us": us_q,
            "torch_producer_then_quant_us": us_t}
        del xs, xqs, y
        torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by rows or columns with no communication; "
              "multi-GPU timing is out of scope)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.profile_linear:
        profile_linear(args.profile_linear, args.steps, args.warmup)
        return

    import numpy as np
    import torch

    import w8a8_int8_dynamic_quant_amd as w8
    from synth_inputs import DIT_BLOCK, make_linear_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w8.lib()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    print("[bench] generating inputs", file=sys.stderr, flush=True)
    inputs = {name: make_linear_inputs(name) for name in DIT_BLOCK}
    layers = []
    for name in DIT_BLOCK:
        d = inputs[name]
        M, K, N = d["M"], d["K"], d["N"]
        wq, sw = w8.quantize_weights(to_dev(d["w"]))            # load time, untimed
        layers.append({
            "name": name, "M": M, "K": K, "N": N,
            "x": to_dev(d["x"]), "wq": wq, "sw": sw,
            "bias": None if d["bias"] is None else to_dev(d["bias"]),
            "xq": torch.empty((M, K), dtype=torch.int8, device=dev),
            "sa": torch.empty((M,), dtype=torch.float32, device=dev),
            "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            "ws": torch.empty((w8.workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev),
            "path": w8.linear_path(M, K, N),
            # w8a8_linear on the GEMM path launches the quantisation and then
            # the product, exactly the two entry points below, unless it
            # splits K (a workspace larger than xq + a_scale): time such a
            # layer through w8a8_linear itself
            "two_call": (w8.linear_path(M, K, N) == w8.PATH_GEMM and
                         w8.workspace_bytes(M, K, N) == align256(M * K) + align256(4 * M)),
        })
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    hev = HipEvents()
    sp = stream.cuda_stream

    def step(gemm_events=None, all_events=None):
        """One pass over the block. gemm_events[i] = (start, end) bracket the
        GEMM launch of layer i; all_events[i] = (a, b, c) bracket layer i's
        quantisation (a..b) and GEMM or fused small-M kernel (b..c)."""
        for i, L in enumerate(layers):
            e = all_events[i] if all_events is not None else None
            if L["two_call"]:
                # w8a8_linear on this path launches exactly these two kernels;
                # calling the two entry points lets events bracket each one.
                if e is not None:
                    hev.record(e[0], sp)
                st = w8.lib().w8a8_quant_act(
                    L["x"].data_ptr(), L["M"], L["K"], L["K"], L["xq"].data_ptr(),
                    L["sa"].data_ptr(), sp)
                if e is not None:
                    hev.record(e[1], sp)
                if gemm_events is not None:
                    hev.record(gemm_events[i][0], sp)
                st |= w8.lib().w8a8_scaled_mm(
                    L["xq"].data_ptr(), L["sa"].data_ptr(), L["M"], L["K"], L["wq"].data_ptr(),
                    L["sw"].data_ptr(), L["N"],
                    None if L["bias"] is None else L["bias"].data_ptr(),
                    L["out"].data_ptr(), L["N"], None, sp)
                if gemm_events is not None:
                    hev.record(gemm_events[i][1], sp)
                if e is not None:
                    hev.record(e[2], sp)
            else:
                if e is not None:
                    hev.record(e[0], sp)
                    hev.record(e[1], sp)
                st = w8.lib().w8a8_linear(
                    L["x"].data_ptr(), L["M"], L["K"], L["K"], L["wq"].data_ptr(),
                    L["sw"].data_ptr(), L["N"],
                    None if L["bias"] is None else L["bias"].data_ptr(),
                    L["out"].data_ptr(), L["N"], L["ws"].data_ptr(), L["ws"].numel(), None, sp)
                if e is not None:
                    hev.record(e[2], sp)
            if st != 0:
                raise RuntimeError(f"{L['name']}: libw8a8 status {st}")

    def new_events(n):
        return [tuple(hev.new() for _ in range(n)) for _ in layers]

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: events (device-scope release) bracket only the GEMM
    # launches, the ones the roofline needs.
    gev = [new_events(2) for _ in range(args.steps)]
    print("[bench] timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(gemm_events=gev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-layer breakdown, after the timed region: events around every launch.
    n_bd = min(args.steps, 20)
    aev = [new_events(3) for _ in range(n_bd)]
    print("[bench] per-layer breakdown", file=sys.stderr, flush=True)
    for s in range(n_bd):
        step(all_events=aev[s])
    torch.cuda.synchronize()

    print("[bench] clock pass", file=sys.stderr, flush=True)
    sclk = clock_pass(step, torch)

    ops_step = sum(2 * L["M"] * L["N"] * L["K"] for L in layers)
    per_shape = []
    gemm_ops = gemm_ms = 0.0
    gemm_launches = 0
    for i, L in enumerate(layers):
        qs = [hev.ms(aev[s][i][0], aev[s][i][1]) for s in range(n_bd)]
        ks = [hev.ms(aev[s][i][1], aev[s][i][2]) for s in range(n_bd)]
        q_ms, k_ms = float(np.mean(qs)), float(np.mean(ks))
        tot = q_ms + k_ms
        M, K, N = L["M"], L["K"], L["N"]
        ops = 2 * M * N * K
        alg_bytes = 2 * M * K + N * K + 4 * N + (2 * N if L["bias"] is not None else 0) + 2 * M * N
        row = {"shape": L["name"], "M": M, "K": K, "N": N,
               "path": "gemm" if L["path"] == w8.PATH_GEMM else "small_m",
               "us": tot * 1e3, "tops": ops / (tot * 1e-3) / 1e12,
               "pct_int8_peak": 100 * ops / (tot * 1e-3) / 1e12 / PEAK_INT8_TOPS,
               "gbs": alg_bytes / (tot * 1e-3) / 1e9,
               "pct_hbm": 100 * alg_bytes / (tot * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "us_median": float(np.median(np.add(qs, ks))) * 1e3}
        if L["two_call"]:
            g_ms = float(np.mean([hev.ms(gev[s][i][0], gev[s][i][1]) for s in range(args.steps)]))
            row["quant_us"] = q_ms * 1e3
            row["quant_gbs"] = (3 * M * K + 4 * M) / (q_ms * 1e-3) / 1e9
            row["gemm_us"] = g_ms * 1e3
            row["gemm_tops"] = ops / (g_ms * 1e-3) / 1e12
            row["gemm_tile"] = list(w8.gemm_tile(M, K, N))
            gemm_ops += ops
            gemm_ms += g_ms
            gemm_launches += 1
        per_shape.append(row)

    hev.close()
    achieved = gemm_ops / (gemm_ms * 1e-3) / 1e12
    counters = load_counters()
    roofline = {
        "bound": "mfma",
        "kernel": GEMM_KERNEL,
        "achieved": achieved,
        "peak": PEAK_INT8_TOPS,
        "unit": "TOPS",
        "frac": achieved / PEAK_INT8_TOPS,
        "traffic": counters.get("hbm_bytes_per_launch_avg"),
        "avg_launch_us": gemm_ms * 1e3 / gemm_launches,
        "ops_per_launch_avg": gemm_ops / gemm_launches,
        "timing": "hipEventReleaseToDevice events around each GEMM launch in the timed region",
    }
    if counters.get("kernel_trace_avg_us"):
        # the same kernel's average duration in the committed rocprofv3
        # kernel trace of this step (no events in that run)
        kt = counters["kernel_trace_avg_us"]
        roofline["kernel_trace"] = {"avg_launch_us": kt,
                                    "achieved": gemm_ops / gemm_launches / (kt * 1e-6) / 1e12,
                                    "frac": gemm_ops / gemm_launches / (kt * 1e-6) / 1e12 /
                                    PEAK_INT8_TOPS,
                                    "source": os.path.relpath(COUNTERS_FILE, ROOT)}
    if sclk is not None:
        # the published peak is quoted at 2.4 GHz; the same MFMA rate at the
        # clock the chip sustained on this step
        sclk["int8_peak_at_mean_mhz_tops"] = PEAK_INT8_TOPS * sclk["mean_mhz"] / 2400.0
        sclk["gemm_frac_at_mean_mhz"] = achieved / sclk["int8_peak_at_mean_mhz_tops"]

    line = {
        "metric": METRIC,
        "value": ops_step / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "dit_block_1024px_w8a8",
                   "linears": [f"{L['M']}x{L['K']}x{L['N']}" for L in layers],
                   "tokens": 4352, "hidden": 3072, "mlp": 12288},
        "roofline": roofline,
        "sclk": sclk,
        "per_shape": per_shape,
        "per_shape_note": ("us/tops/gbs/quant_us: HIP events around every launch in a separate "
                           f"{n_bd}-step pass after the timed region; gemm_us/gemm_tops and "
                           "roofline: events around the GEMM launches inside the timed region"),
    }
    if not args.no_next_rows:
        print("[bench] next rows (W8A16, ingest, fp16, fused producers)", file=sys.stderr, flush=True)
        line["next_rows"] = next_rows(w8, torch, np, dev, to_dev)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        import oracle
        wq_host = {name: oracle.quantize_weights(inputs[name]["w"]) for name in DIT_BLOCK}
        line["cpu_baseline"] = cpu_baseline(inputs, wq_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
