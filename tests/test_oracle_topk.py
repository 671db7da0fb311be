"""Pins of the oracle's index top-k (CPU only).

I_t = top_k over the valid positions ("Compressed sparse attention" page,
"All 25 steps"); selection offset past the window rows and -1 for an absent
entry ("attn_v41.rs" module documentation, SharedV41).  Readings: ties by the
lower position, +0 == -0, -inf and NaN not selectable; the selection is a
set, written in ascending position order.
Pinned by hand-worked cases (tests/golden/topk_hand.txt) and by the defining
invariants checked without sorting: the right count, every selected score >=
every unselected valid score, the threshold group filled from the lowest
positions, nothing invalid selected, and the output order.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from golden_io import kv, lines, num


def check_invariants(s, out, k, offset):
    s = np.asarray(s, dtype=np.float64)
    valid = ~(np.isnan(s) | (s == -np.inf))
    nv = int(valid.sum())
    m = min(k, nv)
    sel = out[:m] - offset
    assert np.all(out[m:] == -1)
    assert len(set(sel.tolist())) == m
    assert np.all(valid[sel])
    if m == 0:
        return
    chosen = np.zeros(s.size, dtype=bool)
    chosen[sel] = True
    rest = valid & ~chosen
    thr = s[sel].min()
    if rest.any():
        assert s[rest].max() <= thr
        # within the threshold group, every chosen position is below every
        # unchosen one
        tie_chosen = np.nonzero(chosen & (s == thr))[0]
        tie_rest = np.nonzero(rest & (s == thr))[0]
        if tie_rest.size:
            assert tie_chosen.max() < tie_rest.min()
    # written in ascending position order
    assert np.all(np.diff(sel) > 0)


def test_hand_cases():
    ls = list(lines("topk_hand.txt"))
    scores = [num(t) for t in ls[0].split(":", 1)[1].split()]
    n = 0
    for ln in ls[1:]:
        spec, want = ln.split(":", 1)[1].split("->")
        k = int(spec.split()[0].split("=")[1])
        off = int(spec.split()[1].split("=")[1])
        got = O.topk(np.array([scores]), k, off)[0]
        assert got.tolist() == [int(v) for v in want.split()]
        n += 1
    assert n == 5


def test_signed_zeros_are_one_value():
    s = np.array([[-0.0, 0.0, -0.0, 0.0, 1.0]])
    assert O.topk(s, 3, 0)[0].tolist() == [0, 1, 4]


@pytest.mark.parametrize("seed", range(20))
def test_invariants_random_with_ties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 300))
    k = int(rng.integers(1, 64))
    s = np.round(rng.standard_normal(L) * 3) / 2           # many ties
    s[rng.uniform(size=L) < 0.1] = -np.inf
    s[rng.uniform(size=L) < 0.05] = np.nan
    z = rng.uniform(size=L) < 0.1
    s[z] = np.where(rng.uniform(size=z.sum()) < 0.5, 0.0, -0.0)
    off = int(rng.integers(0, 200))
    out = O.topk(s[None], k, off)[0]
    check_invariants(s, out, k, off)


def test_brute_force_tiny():
    """All score vectors over {-inf, 0, 1, 2} of length 5, every k: the chosen
    set is the unique m-subset that dominates (score desc, position asc)
    lexicographically, found by enumeration."""
    vals = [-np.inf, 0.0, 1.0, 2.0]
    for sv in itertools.product(vals, repeat=5):
        s = np.array(sv)
        for k in range(1, 6):
            out = O.topk(s[None], k, 0)[0]
            valid = [j for j in range(5) if s[j] != -np.inf]
            m = min(k, len(valid))
            best = None
            for sub in itertools.combinations(valid, m):
                key = sorted(((-s[j], j) for j in sub))
                if best is None or key < best[0]:
                    best = (key, sub)
            want = sorted(j for _, j in best[0]) + [-1] * (k - m)
            assert out.tolist() == want, (sv, k)


def test_fewer_valid_than_k_pads():
    s = np.full((1, 10), -np.inf)
    s[0, [2, 7]] = [0.5, 0.5]
    assert O.topk(s, 4, 100)[0].tolist() == [102, 107, -1, -1]
    assert O.topk(np.full((1, 3), -np.inf), 2, 0)[0].tolist() == [-1, -1]
