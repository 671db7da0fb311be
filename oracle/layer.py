"""Oracle drivers that chain the five steps for one layer (test infrastructure).

prefill: the chunk's kv rows go through the fp8 round trip and become the
window rows (rows_a); the last `window` of them seed the ring; each token gets
its causal window (ascending, -1 padded) and, at ratio > 0, the indexer's
top-k over the compressed rows, offset by the chunk length.
decode: the new kv row goes through the fp8 round trip into ring slot
pos mod window; the query attends over the whole ring oldest first plus the
top-k compressed rows offset by the ring length.

With a RoPE table (rope=(table, rope_dim)), q and the kv rows arrive before
their rotation: q is rotated at its token's position and each kv row is rotated
and then rounded through fp8 (W_{t,448:} <- R_t w; W <- FP8(W)).

Sources: "deepseek_v41_ref::attn" rustdoc (ring example, window_topk_idxs,
sparse_attn, apply_rotary), "Compressed sparse attention" page, "All 25 steps"
(FP8(W), S^I, I_t, J^w_t, Y = [W; Z], J = [J^w; I + |W|], R_t), "attn_v41.rs"
AttnV41Run (rows_a is the chunk at position 0 and the ring otherwise).
"""
from __future__ import annotations

import numpy as np

from . import (WindowCache, fp8_round_rows, indexer_scores, rope_fp8_rows, rope_rows,
               sparse_attn, topk, window_idx)


def prefill(kv_chunk, q, sink, scale, window, ratio=0, latent=None, kI=None,
            qI=None, w=None, cand=None, cand_block=1, k=0, queries=None,
            ring: WindowCache | None = None, rope=None) -> dict:
    T = kv_chunk.shape[0]
    if rope is not None:
        table, rd = rope
        H = q.shape[1]
        q = rope_rows(q, table, np.repeat(np.arange(T), H), rd).reshape(q.shape)
        rows_a = rope_fp8_rows(kv_chunk, table, np.arange(T), rd)
    else:
        rows_a = fp8_round_rows(kv_chunk)
    if ring is not None:
        ring.prefill(rows_a, 0)
    qs = list(range(T) if queries is None else queries)
    widx = window_idx(0, T, window)[qs]
    res = {"rows_a": rows_a, "widx": widx, "q": q}
    if ratio > 0:
        scores = indexer_scores(qI, kI, w, 0, ratio, cand, cand_block, tokens=qs)
        cidx = topk(scores, k, offset=T)
        idx = np.concatenate([widx, cidx], axis=1)
        res.update(scores=scores, cidx=cidx)
    else:
        idx = widx
    res["idx"] = idx
    qsel = np.ascontiguousarray(q[qs])
    res["out"] = sparse_attn(qsel, rows_a, latent if ratio > 0 else None, idx, sink, scale)
    return res


def decode(ring: WindowCache, kv_new, pos, q, sink, scale, ratio=0, latent=None,
           kI=None, qI=None, w=None, cand=None, cand_block=1, k=0, rope=None) -> dict:
    if rope is not None:
        table, rd = rope
        q = rope_rows(q, table, np.full(q.shape[0] * q.shape[1], pos), rd).reshape(q.shape)
        row = rope_fp8_rows(kv_new, table, [pos], rd)
    else:
        row = fp8_round_rows(kv_new)
    slot = ring.put(row[0], pos)
    widx = window_idx(pos, 1, ring.window)
    res = {"row": row, "slot": slot, "widx": widx, "ring": ring.rows.copy(), "q": q}
    if ratio > 0:
        scores = indexer_scores(qI, kI, w, pos, ratio, cand, cand_block)
        cidx = topk(scores, k, offset=ring.window)
        idx = np.concatenate([widx, cidx], axis=1)
        res.update(scores=scores, cidx=cidx)
    else:
        idx = widx
    res["idx"] = idx
    res["out"] = sparse_attn(q, ring.rows, latent if ratio > 0 else None, idx, sink, scale)
    return res
