"""Pins of the oracle's candidate-block selection (CPU only).

What fixes the expected values: the candidate-block top-k selection and the
block-level mask of the "attn_v41" module page and "attn_v41.rs"
(SharedV41.candidates), with the index top-k's ordering rule, and the reading
that a block scores the largest valid score of its positions (parity
unpinned: no page states the block score).  Hand cases, the reduction to the
index top-k at block size 1, brute force, and the selection invariants.
"""
import numpy as np
import pytest

import oracle as O
from golden_io import lines, num

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def hand_cases():
    it = iter(lines("candidate_hand.txt"))
    for ln in it:
        assert ln.startswith("scores:")
        s = [num(t) for t in ln.split(":", 1)[1].split()]
        block = int(next(it).split(":", 1)[1])
        k = int(next(it).split(":", 1)[1])
        mask = [int(t) for t in next(it).split(":", 1)[1].split()]
        yield np.array(s, dtype=np.float64), block, k, mask


def test_hand_cases():
    n = 0
    for s, block, k, mask in hand_cases():
        got = O.candidate_blocks(s[None, :], block, k)[0]
        assert got.tolist() == mask, (s, block, k, got)
        n += 1
    assert n == 5


def block_scores(row, block):
    nb = -(-row.size // block)
    out = np.full(nb, -np.inf)
    for b in range(nb):
        seg = row[b * block:(b + 1) * block]
        seg = seg[~np.isnan(seg)]
        if seg.size:
            out[b] = seg.max()
    return out


def brute(row, block, k):
    bs = block_scores(row, block)
    valid = [b for b in range(bs.size) if bs[b] != -np.inf]
    valid.sort(key=lambda b: (-(bs[b] + 0.0), b))
    mask = np.zeros(bs.size, dtype=np.uint8)
    mask[valid[:k]] = 1
    return mask


@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        n = int(rng.integers(1, 200))
        block = int(rng.integers(1, 12))
        k = int(rng.integers(1, 30))
        row = rng.integers(-4, 5, n).astype(np.float64)       # many ties
        row[rng.random(n) < 0.25] = -np.inf
        row[rng.random(n) < 0.05] = np.nan
        row[row == 0] = np.where(rng.random(int((row == 0).sum())) < 0.5, 0.0, -0.0)
        got = O.candidate_blocks(row[None, :], block, k)[0]
        assert np.array_equal(got, brute(row, block, k)), (seed, n, block, k)


def test_block_size_one_is_the_index_topk():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((5, 300))
    s[:, ::7] = -np.inf
    k = 40
    got = O.candidate_blocks(s, 1, k)
    sel = O.topk(s, k)
    for r in range(5):
        want = np.zeros(300, dtype=np.uint8)
        want[sel[r][sel[r] >= 0]] = 1
        assert np.array_equal(got[r], want)


def test_invariants_large():
    """The decode16-sized case: 32768 positions, blocks of 8, 2048 of 4096."""
    rng = np.random.default_rng(3)
    row = rng.standard_normal(32768).astype(np.float32).astype(np.float64)
    row[20000:] = -np.inf              # causal bound: 2500 visible blocks
    row[::3] = np.round(row[::3], 1)   # ties across blocks
    mask = O.candidate_blocks(row[None, :], 8, 2048)[0]
    bs = block_scores(row, 8)
    valid = bs != -np.inf
    assert mask.sum() == min(2048, int(valid.sum()))
    assert not np.any(mask[~valid])
    chosen, rest = bs[mask == 1], bs[(mask == 0) & valid]
    assert chosen.min() >= rest.max()
    t = chosen.min()
    tied = np.nonzero(bs == t)[0]
    taken = np.nonzero((bs == t) & (mask == 1))[0]
    assert np.array_equal(taken, tied[:taken.size])   # lower blocks first


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.candidate_blocks(np.zeros((1, 8)), 0, 2)
    with pytest.raises(ValueError):
        O.candidate_blocks(np.zeros((1, 8)), 2, 0)
