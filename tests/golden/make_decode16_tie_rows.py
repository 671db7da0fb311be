"""Write decode16_tie_rows.json: for sequences 0-7 of the long-context decode
workload (16 sequences, 32768 compressed rows), the compressed position whose
untied indexer score has rank 400 (0-based; order score desc, position asc).
The ties are then planted by copying that position's index key into 300
other positions, so a group of 301 equal scores straddles the 512th place.
Calls only the oracle and the seeded input generator.

    python tests/golden/make_decode16_tie_rows.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from inputs.workloads import WORKLOADS, decode_sequence  # noqa: E402

RANK = 400


def rank_row(scores: np.ndarray, rank: int) -> int:
    """The position at `rank` (0-based) of the order score desc, position asc.
    np.lexsort sorts by its last key first, so the scores (negated) decide and
    the position breaks ties; the oracle top-k's output is a set written in
    position order and is not a ranking."""
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return int(order[rank])


def source_row(wl, b: int) -> int:
    """Sequence b's rank-RANK position under its untied oracle scores."""
    d = decode_sequence(wl, b, with_ties=False)
    s = O.indexer_scores(d["qI"], d["kI"], d["w"], wl.start_pos, wl.ratio)[0]
    return rank_row(s, RANK)


def main():
    wl = WORKLOADS["decode16"]
    rows = []
    for b in range(8):
        rows.append(source_row(wl, b))
        print(f"sequence {b}: rank-{RANK} position {rows[-1]}", flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode16_tie_rows.json")
    with open(out, "w") as f:
        json.dump({"workload": "decode16", "rank": RANK, "source_rows": rows,
                   "written_by": "tests/golden/make_decode16_tie_rows.py (oracle only)"}, f,
                  indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
