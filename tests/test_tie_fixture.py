"""The long-context decode workload's tie fixture (CPU only).

tests/golden/decode16_tie_rows.json holds, for sequences 0-7, the compressed
position whose untied indexer score has rank 400 in the order score desc,
position asc (the index top-k's order: "Compressed sparse attention" page,
"All 25 steps", I_t, with ties to the lower position).  Copying that
position's index key into 300 others makes 301 equal scores that straddle
the 512th place.  These tests tie the stored rows to their generator and
check that the planted group really straddles the cut in the oracle's top-k.
"""
import json
import os
import sys

import numpy as np

import oracle as O
from inputs.workloads import N_TIE_COPIES, WORKLOADS, decode_sequence, tie_source_rows

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_decode16_tie_rows as MK  # noqa: E402


def test_rank_row_orders_by_score_then_position():
    s = np.array([1.0, 3.0, 2.0, 3.0, 2.0, -0.0, 0.0])
    # order: 3.0 @1, 3.0 @3, 2.0 @2, 2.0 @4, 1.0 @0, -0.0 @5, 0.0 @6
    want = [1, 3, 2, 4, 0, 5, 6]
    assert [MK.rank_row(s, r) for r in range(7)] == want


def test_stored_rows_match_generator():
    with open(os.path.join(HERE, "golden", "decode16_tie_rows.json")) as f:
        stored = json.load(f)
    assert stored["rank"] == MK.RANK
    wl = WORKLOADS["decode16"]
    # sequence 0 (6430) and 1 (32247) recomputed from the oracle
    for b in (0, 1):
        assert MK.source_row(wl, b) == stored["source_rows"][b]


def test_planted_group_straddles_the_cut():
    wl = WORKLOADS["decode16"]
    src = tie_source_rows()[0]
    d = decode_sequence(wl, 0)              # ties planted
    s = O.indexer_scores(d["qI"], d["kI"], d["w"], wl.start_pos, wl.ratio)[0]
    group = np.flatnonzero(s == s[src])
    assert group.size == N_TIE_COPIES + 1
    sel = O.topk(s[None], wl.topk, 0)[0]
    assert np.all(sel >= 0)
    chosen = np.intersect1d(sel, group)
    # some but not all of the group fit: it straddles place 512
    assert 0 < chosen.size < group.size
    # the group is the threshold: everything selected outside it scores higher
    others = np.setdiff1d(sel, group)
    assert np.all(s[others] > s[src])
    # inside the group the lowest positions win
    assert np.array_equal(chosen, np.sort(group)[:chosen.size])
