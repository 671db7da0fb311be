"""Pins of the oracle's indexer score (CPU only).

S^I_{t,j} = sum_h w_{t,h} ReLU(qI_{h,t} . kI_j) over j < floor((t+1)/ratio),
under the block candidate mask ("Compressed sparse attention" page, "All 25
steps").  Pinned by a hand-worked case (tests/golden/indexer_hand.txt), two
special cases that reduce to library matrix products (one head with unit
weight: ReLU of a matmul; non-negative operands: ReLU is the identity and the
score is one matrix-vector product), linearity in w, head-permutation
invariance and the exact -inf pattern of the causal bound and the mask.
"""
import numpy as np
import pytest

import oracle as O
from golden_io import kv
from inputs import synth as S


def bf16(x):
    return S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(h):
    return S.bf16_bits_to_f32(h).astype(np.float64)


def rows_of(s):
    return [[float(v) for v in r.split()] for r in s.split(";")]


def test_hand_case():
    g = kv("indexer_hand.txt")
    qI = bf16(rows_of(g["qI"]))[None]          # [1, HI, DI]
    kI = bf16(rows_of(g["kI"]))
    w = np.array([[float(v) for v in g["w"].split()]], dtype=np.float32)
    want = [float(v) for v in g["S"].split()]
    got = O.indexer_scores(qI, kI, w, start_pos=10 ** 6, ratio=1)
    assert got[0].tolist() == want


def test_one_head_unit_weight_is_relu_matmul():
    rng = np.random.default_rng(0)
    T, L, DI = 5, 40, 64
    qI = bf16(rng.standard_normal((T, 1, DI)))
    kI = bf16(rng.standard_normal((L, DI)))
    w = np.ones((T, 1), dtype=np.float32)
    got = O.indexer_scores(qI, kI, w, start_pos=10 ** 6, ratio=1)
    want = np.maximum(f64(qI[:, 0, :]) @ f64(kI).T, 0.0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_nonnegative_operands_reduce_to_gemv():
    rng = np.random.default_rng(1)
    T, L, HI, DI = 3, 33, 8, 32
    qI = bf16(np.abs(rng.standard_normal((T, HI, DI))))
    kI = bf16(np.abs(rng.standard_normal((L, DI))))
    w = rng.uniform(0, 1, (T, HI)).astype(np.float32)
    got = O.indexer_scores(qI, kI, w, start_pos=10 ** 6, ratio=1)
    for t in range(T):
        v = w[t].astype(np.float64) @ f64(qI[t])          # [DI]
        np.testing.assert_allclose(got[t], f64(kI) @ v, rtol=1e-12)


def test_linear_in_weights_and_head_order():
    rng = np.random.default_rng(2)
    T, L, HI, DI = 2, 20, 4, 32
    qI = bf16(rng.standard_normal((T, HI, DI)))
    kI = bf16(rng.standard_normal((L, DI)))
    w1 = rng.integers(0, 8, (T, HI)).astype(np.float32)
    w2 = rng.integers(0, 8, (T, HI)).astype(np.float32)
    s1 = O.indexer_scores(qI, kI, w1, 10 ** 6, 1)
    s2 = O.indexer_scores(qI, kI, w2, 10 ** 6, 1)
    s12 = O.indexer_scores(qI, kI, w1 + w2, 10 ** 6, 1)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-12)
    perm = rng.permutation(HI)
    sp = O.indexer_scores(qI[:, perm], kI, w1[:, perm], 10 ** 6, 1)
    np.testing.assert_allclose(sp, s1, rtol=1e-12)
    # negating every query head makes a ReLU of the opposite sign: scores add
    # to sum_h w_h |qI_h . kI_j|
    sn = O.indexer_scores((qI ^ np.uint16(0x8000)), kI, w1, 10 ** 6, 1)
    absdot = np.abs(np.einsum("thd,jd->thj", f64(qI), f64(kI)))
    want = np.einsum("th,thj->tj", w1.astype(np.float64), absdot)
    np.testing.assert_allclose(s1 + sn, want, rtol=1e-12)


@pytest.mark.parametrize("start_pos,T,ratio,L", [(0, 12, 4, 4), (0, 64, 4, 16),
                                                 (4095, 1, 4, 1024), (1000, 1, 2, 600)])
def test_causal_bound(start_pos, T, ratio, L):
    rng = np.random.default_rng(3)
    qI = bf16(rng.standard_normal((T, 2, 32)))
    kI = bf16(rng.standard_normal((L, 32)))
    w = np.ones((T, 2), dtype=np.float32)
    s = O.indexer_scores(qI, kI, w, start_pos, ratio)
    for t in range(T):
        n = min(L, (start_pos + t + 1) // ratio)
        assert np.all(np.isfinite(s[t, :n]))
        assert np.all(s[t, n:] == -np.inf)


def test_candidate_mask_blocks():
    rng = np.random.default_rng(4)
    T, L, blk = 6, 64, 8
    qI = bf16(rng.standard_normal((T, 2, 32)))
    kI = bf16(rng.standard_normal((L, 32)))
    w = np.ones((T, 2), dtype=np.float32)
    cand = (rng.uniform(size=(T, L // blk)) < 0.5).astype(np.uint8)
    full = O.indexer_scores(qI, kI, w, 10 ** 6, 1)
    masked = O.indexer_scores(qI, kI, w, 10 ** 6, 1, cand=cand, cand_block=blk)
    for t in range(T):
        keep = np.repeat(cand[t].astype(bool), blk)
        assert np.array_equal(masked[t][keep], full[t][keep])
        assert np.all(masked[t][~keep] == -np.inf)
