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

import concurrent.futures as _cf
import os
import threading

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

_CHUNK = 1 << 16


class _Work:
    """Reused scratch arrays for one chunk (fresh memory is slow to touch)."""

    def __init__(self, n: int = _CHUNK):
        self.i = np.empty(n, dtype=np.uint64)
        self.z = np.empty(n, dtype=np.uint64)
        self.t = np.empty(n, dtype=np.uint64)
        self.f = np.empty(n, dtype=np.float64)


_tls = threading.local()
_PAR_MIN = 1 << 21
_PAR_BLOCK = 1 << 20
_pool = None


def _drop_pool_after_fork() -> None:
    """A forked child inherits the pool object but not its threads: start a
    new one there when needed."""
    global _pool
    _pool = None


os.register_at_fork(after_in_child=_drop_pool_after_fork)


def _w() -> _Work:
    w = getattr(_tls, "work", None)
    if w is None:
        w = _tls.work = _Work()
    return w


def _parallel(n: int, fn) -> None:
    """Run fn(e0, e1) over [0, n) in blocks, on a few threads when n is large
    (numpy releases the GIL inside its loops)."""
    global _pool
    if n < _PAR_MIN:
        fn(0, n)
        return
    if _pool is None:
        _pool = _cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1))
    futs = [_pool.submit(fn, e0, min(n, e0 + _PAR_BLOCK)) for e0 in range(0, n, _PAR_BLOCK)]
    for f in futs:
        f.result()


def _mix64(z: np.ndarray, t: np.ndarray | None = None) -> np.ndarray:
    """SplitMix64 finaliser, in place on z (t: scratch of the same shape)."""
    if t is None:
        t = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.right_shift(z, _S30, out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, _M1, out=z)
        np.right_shift(z, _S27, out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, _M2, out=z)
        np.right_shift(z, _S31, out=t)
        np.bitwise_xor(z, t, out=z)
    return z


def _state0(seed: int, tag: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.array([seed], dtype=np.uint64) * GOLDEN2 + np.uint64(tag)
    return _mix64(s)[0]


def _uniform_chunk(s0: np.uint64, start: int, n: int, w: _Work) -> np.ndarray:
    """Uniforms of elements start .. start+n-1 into w.f[:n]."""
    i, z, t, f = w.i[:n], w.z[:n], w.t[:n], w.f[:n]
    i[:] = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        np.multiply(i, GAMMA, out=z)
        np.add(z, s0, out=z)
    _mix64(z, t)
    np.right_shift(z, _S11, out=z)
    f[:] = z
    f *= 1.0 / 9007199254740992.0
    return f


def stream_u64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """Elements start .. start+n-1 of the SplitMix64 stream (seed, tag)."""
    s0 = _state0(seed, tag)
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = i * GAMMA + s0
    return _mix64(z)


def uniform(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """U[0, 1) doubles from the top 53 bits."""
    s0 = _state0(seed, tag)
    out = np.empty(n, dtype=np.float64)

    def run(e0, e1):
        w = _w()
        for c0 in range(e0, e1, _CHUNK):
            c1 = min(e1, c0 + _CHUNK)
            out[c0:c1] = _uniform_chunk(s0, start + c0, c1 - c0, w)

    _parallel(n, run)
    return out


def _normal_into(seed: int, tag: int, out: np.ndarray, as_bf16: bool = False) -> None:
    """N(0, 1) values into `out` (any float dtype, or uint16 bf16 bits when
    as_bf16): Box-Muller on uniform pairs, element 2p = r cos(theta), element
    2p+1 = r sin(theta)."""
    n = out.shape[0]
    s0 = _state0(seed, tag)
    npair = (n + 1) // 2
    half = _CHUNK // 2

    def run(q0, q1):  # pairs q0 .. q1-1
        w = _w()
        for p0 in range(q0, q1, half):
            p1 = min(q1, p0 + half)
            m = p1 - p0
            u = _uniform_chunk(s0, 2 * p0, 2 * m, w)
            u1 = 1.0 - u[0::2]  # (0, 1]: log is finite
            u2 = u[1::2]
            r = np.sqrt(-2.0 * np.log(u1))
            th = 2.0 * np.pi * u2
            e0 = 2 * p0
            e1 = min(n, 2 * p1)
            z = np.empty(2 * m, dtype=np.float64)
            z[0::2] = r * np.cos(th)
            z[1::2] = r * np.sin(th)
            if as_bf16:
                out[e0:e1] = f32_to_bf16_bits(z[:e1 - e0].astype(np.float32))
            else:
                out[e0:e1] = z[:e1 - e0]

    _parallel(npair, run)


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """N(0, 1) doubles: Box-Muller on uniform pairs (cos, then sin)."""
    out = np.empty(n, dtype=np.float64)
    _normal_into(seed, tag, out)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(seed: int, tag: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _normal_into(seed, tag, out)
    return out.reshape(shape)


def normal_bf16(seed: int, tag: int, shape) -> np.ndarray:
    """bf16 bits of binary32 N(0, 1) values (rounded twice: f64 -> f32 -> bf16)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _normal_into(seed, tag, out, as_bf16=True)
    return out.reshape(shape)


def uniform_f32(seed: int, tag: int, shape, scale: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return (uniform(seed, tag, n) * scale).astype(np.float32).reshape(shape)


def unit_pairs_f32(seed: int, tag: int, shape) -> np.ndarray:
    """f32 [*shape, 2]: random points of the unit circle (a normal pair divided
    by its length in double, then rounded to binary32), for tests of a rotation
    with an arbitrary table."""
    n = int(np.prod(shape))
    z = normal(seed, tag, 2 * n).reshape(n, 2)
    r = np.hypot(z[:, 0], z[:, 1])
    r[r == 0.0] = 1.0
    return (z / r[:, None]).astype(np.float32).reshape(tuple(shape) + (2,))


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
