"""Readers for the hand-built fixtures under tests/golden/.

The byte builder here is written independently of both the oracle's parser and the
input generators' packer (it uses ``struct``), so a layout mistake in either of them
cannot cancel out against it.
"""

from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _q_values(spec: str):
    kind, _, rest = spec.partition(":")
    if kind == "c":
        return [int(rest)] * 32
    if kind == "r":
        a = int(rest)
        return [i + a for i in range(32)]
    if kind == "alt":
        v = int(rest)
        return [v if i % 2 == 0 else -v for i in range(32)]
    if kind == "one":
        p, v = rest.split(":")
        q = [0] * 32
        q[int(p)] = int(v)
        return q
    raise ValueError(spec)


def block_bytes(spec: str) -> bytes:
    """'d=<hex>/<q spec>' -> 34 bytes: little-endian binary16 bits, then 32 int8."""
    dpart, qspec = spec.split("/")
    assert dpart.startswith("d=")
    dbits = int(dpart[2:], 16)
    q = _q_values(qspec)
    assert all(-128 <= v <= 127 for v in q)
    return struct.pack("<H", dbits) + struct.pack("<32b", *q)


def half_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of a binary16 bit pattern (finite values only)."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    assert exp != 0x1F
    if exp == 0:
        return sign * Fraction(man, 1 << 24)
    return sign * Fraction(1024 + man, 1024) * (Fraction(2) ** (exp - 15))


def x_row(spec: str, k: int):
    kind, _, rest = spec.partition(":")
    if kind == "c":
        if "@" in rest:
            v, n = rest.split("@")
            return [float(v) if i < int(n) else 0.0 for i in range(k)]
        return [float(rest)] * k
    if kind == "r":
        a = float(rest)
        return [i + a for i in range(k)]
    if kind == "rev":
        c = float(rest)
        return [c - i for i in range(k)]
    if kind == "one":
        p, v = rest.split(":")
        x = [0.0] * k
        x[int(p)] = float(v)
        return x
    raise ValueError(spec)


def _exact(s: str) -> Fraction:
    return Fraction(s.strip())


def load_linear_cases():
    cases = []
    with open(os.path.join(GOLDEN, "q8_hand_blocks.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, k, wrows, xrows, expect = [t.strip() for t in line.split("|")]
            k = int(k)
            rows = [r.strip() for r in wrows.split(";")]
            wbytes = b"".join(block_bytes(b.strip()) for r in rows for b in r.split(","))
            x = [x_row(s.strip(), k) for s in xrows.split(";")]
            y = [[_exact(v) for v in r.split(",")] for r in expect.split(";")]
            cases.append(dict(name=name, k=k, n=len(rows), w=wbytes, x=x, y=y))
    return cases


def _eval(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "exp": math.exp}))


def load_swiglu_router_cases():
    fused, route = [], []
    with open(os.path.join(GOLDEN, "swiglu_router_hand.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [t.strip() for t in line.split("|")]
            if parts[0] == "fused":
                _, name, k, gate, up, xs, expect = parts
                k = int(k)
                fused.append(dict(name=name, k=k, w=block_bytes(gate) + block_bytes(up),
                                  x=[x_row(xs, k)], h=_eval(expect)))
            elif parts[0] == "route":
                _, name, wr, xs, k, norm, idx, wts = parts
                route.append(dict(
                    name=name,
                    w_router=[[float(v) for v in r.split(",")] for r in wr.split(";")],
                    x=[[float(v) for v in r.split(",")] for r in xs.split(";")],
                    k=int(k), normalize=bool(int(norm)),
                    idx=[[int(v) for v in r.split(",")] for r in idx.split(";")],
                    w=[[_eval(v) for v in r.split(",")] for r in wts.split(";")]))
            else:
                raise ValueError(line)
    return fused, route


def load_act_quant_cases(path=None):
    """Cases of tests/golden/q8_act_hand.txt: dicts with x (32 floats), q (32 ints), dx."""
    path = path or os.path.join(GOLDEN, "q8_act_hand.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, *rest = line.split()
        if head == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif head == "x":
            vals = [float(v) for v in rest]
            cur["x"] = vals + [0.0] * (32 - len(vals))
        elif head == "q":
            vals = [int(v) for v in rest]
            cur["q"] = vals + [0] * (32 - len(vals))
        elif head == "dx":
            cur["dx"] = float(rest[0])
    return cases


def load_q4_0_cases(path=None):
    """Cases of tests/golden/q4_0_hand.txt: dicts with name, bytes (18 uint8), w (32 floats)."""
    path = path or os.path.join(GOLDEN, "q4_0_hand.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, *rest = line.split()
        if head == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif head == "bytes":
            cur["bytes"] = bytes(int(v, 16) for v in rest)
        elif head == "w":
            cur["w"] = [float(v) for v in rest]
    return cases


def _rle(tokens, conv):
    out = []
    for t in tokens:
        if "x" in t:
            v, n = t.rsplit("x", 1)
            out.extend([conv(v)] * int(n))
        else:
            out.append(conv(t))
    return out


def load_k_quant_cases(path=None):
    """Cases of tests/golden/k_quants_hand.txt: dicts with name, format ('q4_k' or 'q6_k'),
    bytes (144 or 210), w (256 floats)."""
    path = path or os.path.join(GOLDEN, "k_quants_hand.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, *rest = line.split()
        if head == "case":
            cur = {"name": rest[0], "format": rest[1]}
            cases.append(cur)
        elif head == "bytes":
            cur["bytes"] = bytes(_rle(rest, lambda v: int(v, 16)))
        elif head == "w":
            cur["w"] = _rle(rest, float)
    return cases
