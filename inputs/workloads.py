"""The synthetic workloads: shapes, seeds and per-sequence input arrays.

Five workloads, named for what they are:
  tiny      ratio-0 + ratio-4 layer pair: a 12-token prefill at position 0,
            then decode steps 12 and 13 through one 8-slot ring; 4 heads x 64,
            compressed cache of 4 rows (3 ever visible), indexer 2 heads x 32,
            top-2.
  decode1   1 sequence at position 4095 (1024 compressed rows).
  decode64  64 sequences at position 32767 (8192 compressed rows each).
  prefill   one 2048-token chunk at position 0, ratio 4 (512 compressed rows),
            block candidate mask.
  decode16  16 sequences at position 131071 (32768 compressed rows) with
            adversarial equal-score ties in sequences 0-11.

Layer geometry of the large workloads: 64 heads x 512, window 128, indexer 64
heads x 128, top-512, ratio 4, sink N(0,1), softmax scale 1/sqrt(512) held as
binary32; RoPE on the last 64 values of each q and kv row with base 10000 (the
last 16 in the tiny pair) when the rotary epilogue is part of the step.  Seeds: 0x5EED0000 + 1000 * workload_id + sequence.

Every array is raw: bf16 values as uint16 bits, f32 as float32.  The kv rows
that the method rounds through fp8 come out unrounded here; whoever consumes
them applies the rounding (the GPU path in the bench, the oracle in tests).
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field

import numpy as np

from . import synth as S

SEED_BASE = 0x5EED0000


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    mode: str            # "decode" | "prefill" | "tiny"
    batch: int
    n_tokens: int        # tokens per sequence in one call (1 for decode)
    start_pos: int
    n_heads: int = 64
    head_dim: int = 512
    window: int = 128
    index_heads: int = 64
    index_dim: int = 128
    topk: int = 512
    ratio: int = 4
    n_rows: int = 0      # L: compressed rows present per sequence
    w_scale: float = 1.0 / 64.0
    cand_block: int = 0  # 0 = no candidate mask
    cand_width: int = 0
    ties: bool = False
    rope_dim: int = 64            # rotated tail of each q / kv row (rope_head_dim)
    rope_theta: float = 10000.0   # ratio-0 table base (rope_theta)

    def seed(self, seq: int) -> int:
        return SEED_BASE + 1000 * self.wid + seq

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the binary32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def window_cols(self) -> int:
        if self.start_pos == 0:
            return min(self.n_tokens, self.window)
        return self.window

    @property
    def width(self) -> int:
        return self.window_cols + (self.topk if self.ratio > 0 else 0)

    @property
    def rows_a_len(self) -> int:
        """Window rows: the chunk's own rows at position 0, else the ring."""
        return self.n_tokens if self.start_pos == 0 else self.window

    @property
    def queries(self) -> int:
        return self.batch * self.n_tokens


WORKLOADS = {
    "decode1": Workload(1, "decode1", "decode", batch=1, n_tokens=1,
                        start_pos=4095, n_rows=1024),
    "decode64": Workload(2, "decode64", "decode", batch=64, n_tokens=1,
                         start_pos=32767, n_rows=8192),
    "prefill": Workload(3, "prefill", "prefill", batch=1, n_tokens=2048,
                        start_pos=0, n_rows=512, cand_block=64, cand_width=8),
    "decode16": Workload(4, "decode16", "decode", batch=16, n_tokens=1,
                         start_pos=131071, n_rows=32768, ties=True),
}

# The tiny pair: layer 0 has ratio 0 (window only), layer 1 ratio 4.
TINY = Workload(0, "tiny", "tiny", batch=1, n_tokens=12, start_pos=0,
                n_heads=4, head_dim=64, window=8, index_heads=2, index_dim=32,
                topk=2, ratio=4, n_rows=4, w_scale=1.0, rope_dim=16)
TINY_DECODE_POSITIONS = (12, 13)


def decode_sequence(wl: Workload, b: int, with_ties: bool = True) -> dict:
    """Inputs of one sequence of a decode workload (one new token at start_pos).
    with_ties=False returns the long-context workload's keys before the ties
    are planted."""
    s = wl.seed(b)
    H, D, W = wl.n_heads, wl.head_dim, wl.window
    HI, DI, L = wl.index_heads, wl.index_dim, wl.n_rows
    d = {
        # ring rows of tokens start_pos-W+1 .. start_pos-1 (unrounded), slot
        # t mod W; the slot of start_pos is overwritten by the new row.
        "ring_raw": S.normal_bf16(s, S.TAG_KV_RING, (W, D)),
        "kv_new": S.normal_bf16(s, S.TAG_KV_NEW, (1, D)),
        "latent": S.normal_bf16(s, S.TAG_LATENT, (L, D)),
        "kI": S.normal_bf16(s, S.TAG_KI, (L, DI)),
        "qI": S.normal_bf16(s, S.TAG_QI, (1, HI, DI)),
        "w": S.uniform_f32(s, S.TAG_W, (1, HI), scale=wl.w_scale),
        "q": S.normal_bf16(s, S.TAG_Q, (1, H, D)),
    }
    if wl.ties and with_ties:
        apply_ties(wl, b, d["kI"])
    return d


def layer_sink(wl: Workload, layer: int = 0) -> np.ndarray:
    return S.normal_f32(wl.seed(0), S.TAG_SINK + 100 * layer, (wl.n_heads,))


# ----------------------------------------------------------------------------
# Adversarial ties of the long-context workload (sequences 0-11)
# ----------------------------------------------------------------------------

_TIE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "tests", "golden", "decode16_tie_rows.json")
N_TIE_COPIES = 300
N_ZERO_KEEP = 300


def tie_source_rows() -> list[int]:
    """Per sequence 0-7: the compressed position whose untied oracle score has
    rank 400 (0-based, order score desc then position asc).  Written once by
    tests/golden/make_decode16_tie_rows.py from the oracle."""
    with open(_TIE_FILE) as f:
        return [int(v) for v in json.load(f)["source_rows"]]


def apply_ties(wl: Workload, b: int, kI: np.ndarray, source_rows=None) -> None:
    """Sequences 0-7: copy the index key of one position into 300 other random
    positions, so 301 positions share one score.  Sequences 8-11: zero every
    index key but 300 random ones, so ~32k positions score 0.  In place."""
    s = wl.seed(b)
    L = kI.shape[0]
    if b < 8:
        rows = tie_source_rows() if source_rows is None else source_rows
        src = rows[b]
        dst = S.choose_distinct(s, S.TAG_TIES, N_TIE_COPIES, L, exclude=src)
        kI[dst] = kI[src]
    elif b < 12:
        keep = S.choose_distinct(s, S.TAG_ZERO_KEEP, N_ZERO_KEEP, L)
        mask = np.ones(L, dtype=bool)
        mask[keep] = False
        kI[mask] = 0


def prefill_inputs(wl: Workload) -> dict:
    s = wl.seed(0)
    T, H, D = wl.n_tokens, wl.n_heads, wl.head_dim
    HI, DI, L = wl.index_heads, wl.index_dim, wl.n_rows
    return {
        "kv_chunk": S.normal_bf16(s, S.TAG_KV_CHUNK, (T, D)),
        "latent": S.normal_bf16(s, S.TAG_LATENT, (L, D)),
        "kI": S.normal_bf16(s, S.TAG_KI, (L, DI)),
        "qI": S.normal_bf16(s, S.TAG_QI, (T, HI, DI)),
        "w": S.uniform_f32(s, S.TAG_W, (T, HI), scale=wl.w_scale),
        "q": S.normal_bf16(s, S.TAG_Q, (T, H, D)),
        "cand": S.bernoulli_u8(s, S.TAG_CAND, (T, wl.cand_width), 0.5),
    }


def tiny_inputs(layer: int) -> dict:
    """The tiny pair.  layer 0: ratio 0 (window only); layer 1: ratio 4 with a
    4-row compressed cache and a 2-head x 32 indexer."""
    wl = TINY
    s = wl.seed(0)
    t0 = 100 * layer
    T, H, D = wl.n_tokens, wl.n_heads, wl.head_dim
    d = {
        "kv_chunk": S.normal_bf16(s, t0 + S.TAG_KV_CHUNK, (T, D)),
        "q": S.normal_bf16(s, t0 + S.TAG_Q, (T, H, D)),
        "sink": S.normal_f32(s, t0 + S.TAG_SINK, (H,)),
    }
    for i, p in enumerate(TINY_DECODE_POSITIONS):
        d[f"kv_new_{p}"] = S.normal_bf16(s, t0 + S.TAG_KV_NEW + 20 * (i + 1), (1, D))
        d[f"q_{p}"] = S.normal_bf16(s, t0 + S.TAG_Q + 20 * (i + 1), (1, H, D))
    if layer == 1:
        HI, DI, L = wl.index_heads, wl.index_dim, wl.n_rows
        d["latent"] = S.normal_bf16(s, t0 + S.TAG_LATENT, (L, D))
        d["kI"] = S.normal_bf16(s, t0 + S.TAG_KI, (L, DI))
        d["qI"] = S.normal_bf16(s, t0 + S.TAG_QI, (T, HI, DI))
        d["w"] = S.uniform_f32(s, t0 + S.TAG_W, (T, HI), scale=wl.w_scale)
        for i, p in enumerate(TINY_DECODE_POSITIONS):
            d[f"qI_{p}"] = S.normal_bf16(s, t0 + S.TAG_QI + 20 * (i + 1), (1, HI, DI))
            d[f"w_{p}"] = S.uniform_f32(s, t0 + S.TAG_W + 20 * (i + 1), (1, HI),
                                        scale=wl.w_scale)
    return d
