"""The score comparison of the GPU parity tests, on the CPU: its second leg,
the binary32 forward error bound, admits what an f32 evaluation of the score
can legitimately differ by on a near-cancelling score, and nothing more."""
import numpy as np
import pytest

import oracle as O
from parity import assert_scores_close, score_abs_bound
from inputs import synth as S


def bf16_bits(x):
    return S.f32_to_bf16_bits(np.asarray(x, np.float32))


def f32_scores(qI, kI, w, t):
    """Score of token t against every key, all in binary32: exact bf16
    products, each dot summed left to right, ReLU, weight, heads summed
    left to right."""
    q = S.bf16_bits_to_f32(qI[t])
    k = S.bf16_bits_to_f32(kI)
    out = np.zeros(k.shape[0], np.float32)
    for j in range(k.shape[0]):
        tot = np.float32(0.0)
        for h in range(q.shape[0]):
            d = np.float32(0.0)
            for x in (q[h] * k[j]).astype(np.float32):
                d = np.float32(d + x)
            tot = np.float32(tot + np.float32(w[t, h] * max(d, np.float32(0.0))))
        out[j] = tot
    return out


def test_f32_scores_of_few_heads_fit_the_bound():
    """Four heads of 32 with one planted cancellation: head 0 of token 0
    against key 3 has the products 1, 2^-25, -1 (exact dot 2^-25), which a
    left-to-right f32 sum turns into 0, so that score leaves the 1e-4
    relative leg entirely and stays inside the forward error bound; the
    random scores of the other keys and tokens pass as well."""
    rng = np.random.default_rng(4)
    T, HI, DI, L = 3, 4, 32, 64
    q = rng.standard_normal((T, HI, DI))
    k = rng.standard_normal((L, DI))
    q[0] = 0.0
    q[0, 0, :3] = [1.0, 2.0 ** -25, -1.0]
    k[3, :3] = 1.0
    qI, kI = bf16_bits(q), bf16_bits(k)
    w = (rng.uniform(0, 1, (T, HI)) / 8).astype(np.float32)
    ora = O.indexer_scores(qI, kI, w, 10 ** 6, 1)
    assert ora[0, 3] == pytest.approx(float(w[0, 0]) * 2.0 ** -25, rel=1e-12)
    got = np.stack([f32_scores(qI, kI, w, t) for t in range(T)]).astype(np.float64)
    assert got[0, 3] == 0.0
    assert_scores_close(got, ora, "f32 evaluation", operands=(qI, kI, w, range(T)))
    with pytest.raises(AssertionError):
        assert_scores_close(got, ora, "f32 evaluation, relative leg only")


def test_bound_does_not_admit_a_wrong_score():
    """An error far past the bound fails, with or without operands; the bound
    itself is the sum of |w q k| written out."""
    rng = np.random.default_rng(5)
    T, HI, DI, L = 2, 64, 128, 50
    qI = bf16_bits(rng.standard_normal((T, HI, DI)))
    kI = bf16_bits(rng.standard_normal((L, DI)))
    w = (rng.uniform(0, 1, (T, HI)) / 64).astype(np.float32)
    ora = O.indexer_scores(qI, kI, w, 10 ** 6, 1)
    q = S.bf16_bits_to_f32(qI[1]).astype(np.float64)
    k = S.bf16_bits_to_f32(kI[7]).astype(np.float64)
    by_hand = sum(float(w[1, h]) * sum(abs(q[h, d] * k[d]) for d in range(DI)) for h in range(HI))
    assert score_abs_bound(qI, kI, w, 1, 7) == pytest.approx(by_hand, rel=1e-12)
    bad = ora.copy()
    bad[1, 7] *= 1.001
    with pytest.raises(AssertionError):
        assert_scores_close(bad, ora, "wrong", operands=(qI, kI, w, range(T)))
    assert_scores_close(ora.copy(), ora, "same", operands=(qI, kI, w, range(T)))
