"""Builds libw8a8.so (HIP, gfx950) in-tree with hipcc.

    python -m w8a8_int8_dynamic_quant_amd.build_lib

First the host program csrc/gen_gelu_table.cpp is built with g++ and run: it
writes _build/gelu_table.inc, the GELU producer's bf16 -> bf16 tables
(GELU in double precision, rounded once to the nearest bf16). Then
every source under csrc/ is compiled to an object under _build/ and linked
into w8a8_int8_dynamic_quant_amd/libw8a8.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw8a8.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # bit-exact numerics: no fused multiply-add, correctly rounded division
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


# The GELU tables are computed in IEEE double precision (no fast-math, no
# contraction) and rounded once to bf16.
GXX_FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def gen_gelu_table(verbose: bool = False, build_dir: str = BUILD) -> str:
    """Builds and runs the GELU table generator; returns the path of the
    gelu_table.inc it wrote under build_dir."""
    gxx = shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found: it builds the GELU table generator")
    os.makedirs(build_dir, exist_ok=True)
    exe = os.path.join(build_dir, "gen_gelu_table")
    out = os.path.join(build_dir, "gelu_table.inc")
    cmd = [gxx, *GXX_FLAGS, os.path.join(CSRC, "gen_gelu_table.cpp"), "-o", exe]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("gen_gelu_table build failed:\n" + r.stdout.decode(errors="replace"))
    r = subprocess.run([exe, out + ".tmp"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("gen_gelu_table failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(out + ".tmp", out)
    return out


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libw8a8")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    gen_gelu_table(verbose)
    cc = hipcc()
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, "-I", BUILD, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text, flush=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
