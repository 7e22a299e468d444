"""Readers for the hand-computed fixtures under tests/golden/."""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _num(tok: str) -> float:
    if "0x" in tok and "p" in tok:
        return float.fromhex(tok)
    return float(tok)


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if line and not line.startswith("#"):
                yield line


def quant_cases():
    """[(x values, scale, q values)]"""
    out = []
    for line in _lines("quant_hand_cases.txt"):
        xs, s, qs = (p.strip() for p in line.split("|"))
        out.append(([_num(t) for t in xs.split()], _num(s), [int(t) for t in qs.split()]))
    return out


def epilogue_cases():
    """[(acc, s_a, s_w, bias_bits or None, y_bits)]"""
    out = []
    for line in _lines("epilogue_hand_cases.txt"):
        lhs, y = (p.strip() for p in line.split("|"))
        acc, sa, sw, b = lhs.split()
        bias = None if b == "-" else int(b, 16)
        out.append((int(acc), _num(sa), _num(sw), bias, int(y, 16)))
    return out


def gemm_case():
    rows = {"xq": [], "wq": [], "acc": []}
    for line in _lines("gemm_hand_case.txt"):
        tag, *vals = line.split()
        rows[tag].append([int(v) for v in vals])
    return rows["xq"], rows["wq"], rows["acc"]


def pack_quantized_cases():
    """[(word as unsigned int, [four int8 values])]"""
    out = []
    for line in _lines("pack_quantized_hand_cases.txt"):
        w, qs = (p.strip() for p in line.split("|"))
        out.append((int(w, 16), [int(t) for t in qs.split()]))
    return out


def w8a16_cases(name="w8a16_hand_cases.txt"):
    """[(x values, wq values, s_w, bias_bits or None, y_bits)]"""
    out = []
    for line in _lines(name):
        xs, ws, s, b, y = (p.strip() for p in line.split("|"))
        out.append(([_num(t) for t in xs.split()], [int(t) for t in ws.split()], _num(s),
                    None if b == "-" else int(b, 16), int(y, 16)))
    return out


def f16_cases():
    """({'quant': [(x values, scale, q values)], 'epi': [(acc, s_a, s_w,
    bias_bits or None, y_bits)]}) from f16_hand_cases.txt."""
    out = {"quant": [], "epi": []}
    for line in _lines("f16_hand_cases.txt"):
        tag, *rest = (p.strip() for p in line.split("|"))
        if tag == "quant":
            xs, s, qs = rest
            out["quant"].append(([_num(t) for t in xs.split()], _num(s),
                                 [int(t) for t in qs.split()]))
        else:
            lhs, y = rest
            acc, sa, sw, b = lhs.split()
            out["epi"].append((int(acc), _num(sa), _num(sw), None if b == "-" else int(b, 16),
                               int(y, 16)))
    return out


def producer_cases():
    """(LN cases [(x, shift, scale, eps, v, q or None)], GELU cases [(z, Phi(z))])"""
    ln, ge = [], []
    for line in _lines("producer_hand_cases.txt"):
        parts = [p.strip() for p in line.split("|")]
        if parts[0] == "LN":
            x, sh, sc, eps, v = ([_num(t) for t in p.split()] for p in parts[1:6])
            q = [int(t) for t in parts[6].split()] if len(parts) > 6 else None
            ln.append((x, sh, sc, eps[0], v, q))
        elif parts[0] == "GELU":
            ge.append((_num(parts[1]), _num(parts[2])))
        else:
            raise ValueError(line)
    return ln, ge
