"""Pins of the oracle's sparse attention with the sink (CPU only).

S = q . g / sqrt(d); A_i = exp S_i / (exp sink + sum_j exp S_j); O = sum A_i g_i
("Compressed sparse attention" page, "All 25 steps", sparse attention; the
sparse_attn contract of the "deepseek_v41_ref::attn" rustdoc: -1 skipped, f32
softmax with the sink in the denominator only, bf16 out).  Pinned by: the
weights plus the sink's share summing to 1; an explicit brute-force softmax
over the logit vector with the sink column, the sink column dropped; closed
forms (one valid row: o = g sigmoid(s - sink); n identical rows: o = g
sigmoid(s + ln n - sink)); the sink -> -inf limit against torch's
scaled-dot-product attention on the CPU; all -1 gives 0; invariance under a
permutation of idx; the joint index space (entries >= rows_a_len read rows_b).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from inputs import synth as S


def bf16(x):
    return S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(h):
    return S.bf16_bits_to_f32(h).astype(np.float64)


def rnd(seed, shape, scale=1.0):
    return bf16(np.random.default_rng(seed).standard_normal(shape) * scale)


def ulps(a, b):
    """|a - b| in bf16 ulps of b (elementwise)."""
    b = np.asarray(b, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -126)))
    return np.abs(np.asarray(a, dtype=np.float64) - b) / 2.0 ** (e - 7)


def test_weights_and_sink_share_sum_to_one():
    D, A, Lb, width = 64, 16, 20, 24
    q = rnd(0, (D,))
    ra, rb = rnd(1, (A, D)), rnd(2, (Lb, D))
    rng = np.random.default_rng(3)
    idx = rng.integers(-1, A + Lb, width).astype(np.int32)
    for sink in (-3.0, 0.0, 2.5):
        w, share = O.attn_weights(q, ra, rb, idx, sink, 0.125)
        assert abs(w.sum() + share - 1.0) < 1e-12
        assert np.all(w[idx < 0] == 0)


def test_brute_force_softmax_with_sink_column():
    D, A, width = 32, 6, 6
    q = rnd(10, (D,))
    ra = rnd(11, (A, D))
    idx = np.array([3, -1, 0, 5, -1, 1], dtype=np.int32)
    sink, scale = float(np.float32(0.7)), 1.0 / math.sqrt(D)   # the sink is binary32
    logits = [sink]
    for i in idx:
        if i >= 0:
            logits.append(scale * sum(f64(q)[d] * f64(ra[i])[d] for d in range(D)))
    mx = max(logits)
    ex = [math.exp(v - mx) for v in logits]
    sm = [v / sum(ex) for v in ex][1:]          # drop the sink column
    w, _ = O.attn_weights(q, ra, None, idx, sink, scale)
    np.testing.assert_allclose(w[idx >= 0], sm, rtol=1e-12)


def test_single_valid_row_closed_form():
    D = 64
    q, g = rnd(20, (D,)), rnd(21, (1, D))
    sink, scale = np.float32(0.3), 0.125
    idx = np.array([[-1, 0, -1]], dtype=np.int32)
    o = O.sparse_attn(q[None, None], g, None, idx, np.array([sink]), scale)[0, 0]
    s = scale * float(f64(q) @ f64(g[0]))
    sig = 1.0 / (1.0 + math.exp(-(s - float(sink))))
    want = f64(g[0]) * sig
    assert np.max(ulps(f64(o), want)) <= 0.5 + 1e-9


def test_identical_rows_closed_form():
    D, n = 64, 37
    q, g = rnd(30, (D,)), rnd(31, (1, D))
    rows = np.repeat(g, n, axis=0)
    sink, scale = np.float32(-1.25), 0.125
    idx = np.arange(n, dtype=np.int32)[None]
    o = O.sparse_attn(q[None, None], rows, None, idx, np.array([sink]), scale)[0, 0]
    s = scale * float(f64(q) @ f64(g[0]))
    sig = 1.0 / (1.0 + math.exp(-(s + math.log(n) - float(sink))))
    want = f64(g[0]) * sig
    assert np.max(ulps(f64(o), want)) <= 0.5 + 1e-6


def test_sink_to_minus_inf_is_textbook_attention():
    T, H, D, A = 3, 4, 64, 40
    q = rnd(40, (T, H, D))
    ra = rnd(41, (A, D))
    rng = np.random.default_rng(42)
    idx = np.stack([rng.permutation(A)[:24] for _ in range(T)]).astype(np.int32)
    sink = np.full(H, -np.inf, dtype=np.float32)
    scale = 1.0 / math.sqrt(D)
    o = O.sparse_attn(q, ra, None, idx, sink, scale)
    for t in range(T):
        G = torch.tensor(f64(ra[idx[t]]))                     # [n, D]
        Q = torch.tensor(f64(q[t]))                           # [H, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], G[None], G[None], scale=scale)[0].numpy()
        assert np.max(ulps(f64(o[t]), ref)) <= 1.0


def test_all_absent_gives_zero():
    q = rnd(50, (2, 4, 64))
    ra = rnd(51, (8, 64))
    idx = np.full((2, 10), -1, dtype=np.int32)
    o = O.sparse_attn(q, ra, None, idx, np.zeros(4, np.float32), 0.125)
    assert np.all(o == 0)


def test_permutation_invariance():
    T, H, D, A = 2, 4, 64, 30
    q = rnd(60, (T, H, D))
    ra = rnd(61, (A, D))
    rng = np.random.default_rng(62)
    idx = np.stack([rng.integers(-1, A, 20) for _ in range(T)]).astype(np.int32)
    sink = rnd(63, (H,)).astype(np.float32) * 0 + np.float32(0.5)
    o1 = O.sparse_attn(q, ra, None, idx, sink, 0.125)
    o2 = O.sparse_attn(q, ra, None, idx[:, rng.permutation(20)], sink, 0.125)
    assert np.max(ulps(f64(o1), f64(o2))) <= 1.0


def test_joint_index_space_and_out_of_range():
    """Entries below rows_a_len read rows_a, the rest rows_b shifted by
    rows_a_len; out-of-range entries are skipped like -1."""
    D, A, Lb = 64, 5, 7
    ra = np.stack([bf16(np.full(D, float(i + 1))) for i in range(A)])
    rb = np.stack([bf16(np.full(D, float(-(i + 1)))) for i in range(Lb)])
    q = bf16(np.zeros((1, 1, D)))
    sink = np.array([-np.inf], dtype=np.float32)
    for ix, want in [(0, 1.0), (4, 5.0), (5, -1.0), (11, -7.0)]:
        idx = np.array([[ix, -1, A + Lb, 10 ** 6]], dtype=np.int32)
        o = O.sparse_attn(q, ra, rb, idx, sink, 0.125)
        assert np.all(f64(o) == want), ix
