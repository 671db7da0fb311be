"""Pins of the oracle's window selection and ring (CPU only).

Fixed by the ring-cache example of the "deepseek_v41_ref::attn" rustdoc
(tests/golden/ring_example.txt), the window_topk_idxs contract on that page,
the window set J^w_t = {max(0, t-127) .. t} of the "Compressed sparse
attention" page and the 128 + 500 = 628 join of the "Join rows" page
(tests/golden/join_count.txt).
"""
import numpy as np
import pytest

import oracle as O
from golden_io import kv


def ints(s):
    return [int(v) for v in s.split()]


def test_ring_example():
    g = kv("ring_example.txt")
    W, T = int(g["window"]), int(g["prefill_tokens"])
    D = 32
    ring = O.WindowCache(W, D)
    rows = np.arange(T * D, dtype=np.uint16).reshape(T, D)
    ring.prefill(rows)
    assert ring.token.tolist() == ints(g["ring_after_prefill"])
    widx = O.window_idx(0, T, W)
    for t in (0, 7, 11):
        assert widx[t].tolist() == ints(g[f"prefill_row_{t}"])
    for p in (12, 13):
        slot = ring.put(np.full(D, p, dtype=np.uint16), p)
        assert slot == int(g[f"decode_{p}_slot"])
        idx = O.window_idx(p, 1, W)[0]
        assert idx.tolist() == ints(g[f"decode_{p}_idx"])
        # oldest first, the current token last
        toks = ring.token[idx]
        assert toks.tolist() == list(range(p - W + 1, p + 1))


@pytest.mark.parametrize("T,W", [(1, 8), (5, 8), (12, 8), (300, 128), (2048, 128)])
def test_prefill_window_is_causal_band(T, W):
    idx = O.window_idx(0, T, W)
    assert idx.shape == (T, min(T, W))
    for t in range(T):
        lo = max(0, t - W + 1)
        want = list(range(lo, t + 1))
        want += [-1] * (idx.shape[1] - len(want))
        assert idx[t].tolist() == want


def test_decode_before_ring_fills():
    W = 8
    for p in range(1, W - 1):
        idx = O.window_idx(p, 1, W)[0]
        assert idx.tolist() == list(range(p + 1)) + [-1] * (W - p - 1)
    # p = W-1: the ring has just filled; slot order 0..W-1 is oldest first
    assert O.window_idx(W - 1, 1, W)[0].tolist() == list(range(W))


def test_decode_wrapped_oldest_first():
    W = 128
    for p in (127, 128, 4095, 32767, 131071, 1000):
        idx = O.window_idx(p, 1, W)[0]
        toks = [(p - W + 1 + c) for c in range(W)]
        assert idx.tolist() == [t % W for t in toks]


def test_decode_takes_one_token():
    with pytest.raises(ValueError):
        O.window_idx(5, 2, 8)


def test_join_count():
    g = kv("join_count.txt")
    p, ratio, W = int(g["position"]), int(g["ratio"]), int(g["window"])
    n = O.causal_count(p, ratio, 10 ** 9)
    assert n == int(g["compressed"])
    assert W + n == int(g["joined"])
    # the cap at the rows present
    assert O.causal_count(p, ratio, 100) == 100
