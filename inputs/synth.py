"""Seeded synthetic inputs shared by the tests, the oracle timing and the bench.

This module draws random numbers and lays them out in the shapes of the
workloads; it holds none of the attention method's arithmetic (no fp8
rounding, no scores, no selection, no softmax).  Both the GPU path and the
CPU oracle read the arrays it returns.

Generator: SplitMix64 used as a counter-based stream.  Element i of the
stream (seed, tag) is mix64(state0 + (i + 1) * GAMMA) with
state0 = mix64(seed * GOLDEN2 + tag), so any slice can be drawn on its own.
Uniforms take the top 53 bits; normals come from Box-Muller on consecutive
uniform pairs; bf16 values are the binary32 value rounded to nearest even.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
GOLDEN2 = np.uint64(0xD1342543DE82EF95)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_S30 = np.uint64(30)
_S27 = np.uint64(27)
_S31 = np.uint64(31)
_S11 = np.uint64(11)

# Stream tags: one per kind of tensor.
TAG_Q = 1
TAG_KV_RING = 2
TAG_KV_NEW = 3
TAG_LATENT = 4
TAG_KI = 5
TAG_QI = 6
TAG_W = 7
TAG_SINK = 8
TAG_CAND = 9
TAG_TIES = 10
TAG_ZERO_KEEP = 11
TAG_KV_CHUNK = 12
TAG_MISC = 13

_CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _S30)) * _M1
        z = (z ^ (z >> _S27)) * _M2
        return z ^ (z >> _S31)


def _state0(seed: int, tag: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.array([seed], dtype=np.uint64) * GOLDEN2 + np.uint64(tag)
    return _mix64(s)[0]


def stream_u64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """Elements start .. start+n-1 of the SplitMix64 stream (seed, tag)."""
    s0 = _state0(seed, tag)
    out = np.empty(n, dtype=np.uint64)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        i = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
        with np.errstate(over="ignore"):
            out[c0:c1] = _mix64(s0 + i * GAMMA)
    return out


def uniform(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """U[0, 1) doubles from the top 53 bits."""
    u = stream_u64(seed, tag, n, start)
    return (u >> _S11).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """N(0, 1) doubles: Box-Muller on uniform pairs (cos, then sin)."""
    npair = (n + 1) // 2
    out = np.empty(2 * npair, dtype=np.float64)
    for p0 in range(0, npair, _CHUNK):
        p1 = min(npair, p0 + _CHUNK)
        u = uniform(seed, tag, 2 * (p1 - p0), start=2 * p0)
        u1 = 1.0 - u[0::2]  # (0, 1]: log is finite
        u2 = u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        th = 2.0 * np.pi * u2
        out[2 * p0:2 * p1:2] = r * np.cos(th)
        out[2 * p0 + 1:2 * p1:2] = r * np.sin(th)
    return out[:n]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tag: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal(seed, tag, n).astype(np.float32)).reshape(shape)


def normal_f32(seed: int, tag: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return normal(seed, tag, n).astype(np.float32).reshape(shape)


def uniform_f32(seed: int, tag: int, shape, scale: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return (uniform(seed, tag, n) * scale).astype(np.float32).reshape(shape)


def bernoulli_u8(seed: int, tag: int, shape, p: float = 0.5) -> np.ndarray:
    n = int(np.prod(shape))
    return (uniform(seed, tag, n) < p).astype(np.uint8).reshape(shape)


def choose_distinct(seed: int, tag: int, n_pick: int, n_total: int,
                    exclude: int | None = None) -> np.ndarray:
    """n_pick distinct positions of range(n_total) (minus `exclude`), sorted:
    a seeded partial Fisher-Yates shuffle."""
    pool = np.arange(n_total, dtype=np.int64)
    if exclude is not None:
        pool = pool[pool != exclude]
    u = uniform(seed, tag, n_pick)
    m = pool.shape[0]
    for i in range(n_pick):
        r = i + int(u[i] * (m - i))
        pool[i], pool[r] = pool[r], pool[i]
    return np.sort(pool[:n_pick])
