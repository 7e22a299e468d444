"""Helpers for the GPU parity tests: host <-> device transfers of bf16 bit
patterns and the comparison rules (bit-exact ints and scales, bf16 within 1
ulp with equal signs of zero)."""
from __future__ import annotations

import sys

import numpy as np
import torch


def announce(msg: str) -> None:
    """Print what the next GPU step is, flushed, before it runs."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    """Maps bf16 bit patterns to integers in value order (+0 and -0 -> 0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_bf16_close(got_bits: np.ndarray, exp_bits: np.ndarray, max_ulp: int = 1) -> dict:
    """Every element within max_ulp bf16 ulps; returns diff statistics."""
    assert got_bits.shape == exp_bits.shape
    d = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(exp_bits))
    stats = {"max_ulp": int(d.max()) if d.size else 0, "n_diff": int(np.count_nonzero(d)),
             "n": int(d.size)}
    assert stats["max_ulp"] <= max_ulp, stats
    return stats


def assert_equal(got, exp, what: str) -> None:
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    if got.dtype.kind == "f":
        ok = np.array_equal(got.view(np.uint32), exp.astype(np.float32).view(np.uint32))
    else:
        ok = np.array_equal(got, exp)
    if not ok:
        bad = np.argwhere(got != exp)
        first = tuple(bad[0]) if bad.size else None
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {first}: "
                             f"got {got[first] if first else None} exp {exp[first] if first else None}")


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16).cuda()
