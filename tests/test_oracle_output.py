"""Pins of the oracle's grouped output projection (CPU only).

What fixes the expected values: the "Grouped output" formulas of the
"Compressed sparse attention" page (o^g = [O_bar_h]_{h in r} W_OA,r, then
o^g W_OB), the model code's per-group contraction (block-diagonal wo_a over
contiguous head groups), the [out, in] layouts of "attn_v41.rs", and the
precision paragraph (f32 accumulation, bf16 results).  A hand case, the
one-group reduction to a plain matrix product, the block-diagonal structure
and the head-to-group assignment.
"""
import numpy as np
import pytest

import oracle as O
from golden_io import kv
from inputs import synth as S


def bf(x):
    return S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(h):
    return S.bf16_bits_to_f32(np.asarray(h, dtype=np.uint16)).astype(np.float64)


def ulp_bf16(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def test_hand_case():
    g = kv("grouped_output_hand.txt")
    groups = int(g["groups"])
    vals = {k: [float(t) for t in v.split()] for k, v in g.items() if k != "groups"}
    o = bf([vals["o_bar"]])
    wa = bf(np.array(vals["wo_a"]).reshape(4, 2))
    wb = bf(np.array(vals["wo_b"]).reshape(2, 4))
    og, x = O.grouped_output(o, wa, wb, groups)
    assert f64(og)[0].tolist() == vals["og"]
    assert f64(x)[0].tolist() == vals["x"]


def test_one_group_is_a_matrix_product():
    T, gw, R, dim = 6, 96, 40, 24
    o = S.normal_bf16(1, S.TAG_Q, (T, gw))
    wa = S.normal_bf16(2, S.TAG_MISC, (R, gw))
    wb = S.normal_bf16(3, S.TAG_MISC, (dim, R))
    og, x = O.grouped_output(o, wa, wb, 1)
    exact = f64(o) @ f64(wa).T
    assert np.all(np.abs(f64(og) - exact) <= 0.5 * ulp_bf16(exact))
    exact_x = f64(og) @ f64(wb).T          # the second projection takes the bf16 og
    assert np.all(np.abs(f64(x) - exact_x) <= 0.5 * ulp_bf16(exact_x))


def test_groups_are_block_diagonal():
    T, G, gw, R, dim = 3, 4, 32, 8, 16
    o = S.normal_bf16(4, S.TAG_Q, (T, G * gw))
    wa = S.normal_bf16(5, S.TAG_MISC, (G * R, gw))
    wb = S.normal_bf16(6, S.TAG_MISC, (dim, G * R))
    og, _ = O.grouped_output(o, wa, wb, G)
    for g in range(G):
        o2 = o.copy()
        other = np.ones(G * gw, dtype=bool)
        other[g * gw:(g + 1) * gw] = False
        o2[:, other] = S.normal_bf16(7 + g, S.TAG_Q, (T, int(other.sum())))
        og2, _ = O.grouped_output(o2, wa, wb, G)
        assert np.array_equal(og2[:, g * R:(g + 1) * R], og[:, g * R:(g + 1) * R])
        # and each group contracts with its own rows of wo_a only
        exact = f64(o[:, g * gw:(g + 1) * gw]) @ f64(wa[g * R:(g + 1) * R]).T
        assert np.all(np.abs(f64(og[:, g * R:(g + 1) * R]) - exact) <= 0.5 * ulp_bf16(exact))


def test_heads_go_to_contiguous_groups():
    """With [T, H, D] output, group g holds heads g*H/G .. (g+1)*H/G - 1."""
    T, H, D, G, R, dim = 1, 8, 16, 4, 2, 3
    wa = bf(np.ones((G * R, H * D // G)))
    wb = bf(np.ones((dim, G * R)))
    for h in range(H):
        o = np.zeros((T, H, D), dtype=np.uint16)
        o[0, h, 5] = bf([1.0])[0]
        og, x = O.grouped_output(o, wa, wb, G)
        expect = np.zeros(G * R)
        expect[(h // (H // G)) * R:(h // (H // G) + 1) * R] = 1.0
        assert f64(og)[0].tolist() == expect.tolist()
        assert f64(x)[0].tolist() == [float(R)] * dim


def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        O.grouped_output(np.zeros((1, 10), np.uint16), np.zeros((4, 4), np.uint16),
                         np.zeros((2, 4), np.uint16), 2)


def test_linear_is_a_matrix_product():
    a = S.normal_bf16(11, S.TAG_Q, (7, 160))
    w = S.normal_bf16(12, S.TAG_MISC, (33, 160))
    y = O.linear_bf16(a, w)
    exact = f64(a) @ f64(w).T
    assert np.all(np.abs(f64(y) - exact) <= 0.5 * ulp_bf16(exact))
    # a hand case: [out, in] weights
    a = bf([[1, 2, 3]])
    w = bf([[1, 0, 0], [0, 1, 1], [2, -1, 4]])
    assert f64(O.linear_bf16(a, w))[0].tolist() == [1.0, 5.0, 12.0]


def test_grouped_output_is_two_linear_projections():
    """Each group's block is a linear_bf16 of its slice, and x is a
    linear_bf16 of the bf16 og (the same rounding points)."""
    T, G, gw, R, dim = 4, 3, 64, 16, 24
    o = S.normal_bf16(13, S.TAG_Q, (T, G * gw))
    wa = S.normal_bf16(14, S.TAG_MISC, (G * R, gw))
    wb = S.normal_bf16(15, S.TAG_MISC, (dim, G * R))
    og, x = O.grouped_output(o, wa, wb, G)
    for g in range(G):
        assert np.array_equal(og[:, g * R:(g + 1) * R],
                              O.linear_bf16(o[:, g * gw:(g + 1) * gw], wa[g * R:(g + 1) * R]))
    assert np.array_equal(x, O.linear_bf16(og, wb))
