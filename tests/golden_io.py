"""Readers for the hand-written fixtures under tests/golden/."""
from __future__ import annotations

import math
import os
import struct

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def kv(name):
    out = {}
    for ln in lines(name):
        k, v = ln.split(":", 1)
        out[k.strip()] = v.strip()
    return out


def num(tok: str) -> float:
    """'p-10' = 2^-10, '3p-24' = 3*2^-24, '-p-32', '-0', decimals, 'inf', 'nan'."""
    tok = tok.strip()
    if tok == "-0":
        return -0.0
    if "p" in tok and not tok.lstrip("-").startswith(("inf", "nan")):
        neg = tok.startswith("-")
        body = tok[1:] if neg else tok
        mant, ex = body.split("p")
        v = (float(mant) if mant else 1.0) * math.ldexp(1.0, int(ex))
        return -v if neg else v
    return float(tok)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def exact_bf16(x: float) -> int:
    """bf16 bits of x; x must be exactly representable."""
    b = f32_bits(x)
    assert struct.unpack("<f", struct.pack("<I", b))[0] == x or math.isnan(x)
    assert b & 0xFFFF == 0, f"{x!r} is not a bf16 value"
    return b >> 16
