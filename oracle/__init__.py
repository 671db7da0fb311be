"""CPU oracle of the compressed-sparse-attention hot path (test infrastructure).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  It wraps the plain C library built from v41_oracle.c (double
precision, scalar loops) with numpy in/out; it shares nothing with the GPU
library.  The citations for each step are in v41_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        u16p = C.POINTER(C.c_uint16)
        f64p = C.POINTER(C.c_double)
        f32p = C.POINTER(C.c_float)
        i32p = C.POINTER(C.c_int32)
        u8p = C.POINTER(C.c_uint8)
        L.ora_bf16_to_double.argtypes = [C.c_uint16]
        L.ora_bf16_to_double.restype = C.c_double
        L.ora_double_to_bf16.argtypes = [C.c_double]
        L.ora_double_to_bf16.restype = C.c_uint16
        L.ora_pow2_ceil.argtypes = [C.c_float]
        L.ora_pow2_ceil.restype = C.c_float
        L.ora_e4m3_round.argtypes = [C.c_double]
        L.ora_e4m3_round.restype = C.c_double
        L.ora_fp8_round_rows.argtypes = [u16p, u16p, C.c_int64, C.c_int32, C.c_int32]
        L.ora_fp8_round_rows.restype = C.c_int
        L.ora_window_idx.argtypes = [C.c_int64, C.c_int32, C.c_int32, i32p]
        L.ora_window_idx.restype = C.c_int
        L.ora_causal_count.argtypes = [C.c_int64, C.c_int32, C.c_int64]
        L.ora_causal_count.restype = C.c_int64
        L.ora_indexer_scores_one.argtypes = [u16p, u16p, f32p, u8p, C.c_int32, C.c_int32,
                                             C.c_int32, C.c_int64, C.c_int64, f64p]
        L.ora_indexer_scores_one.restype = None
        L.ora_topk_one.argtypes = [f64p, C.c_int64, C.c_int32, C.c_int32, i32p]
        L.ora_topk_one.restype = C.c_int64
        L.ora_attn_weights_one_head.argtypes = [u16p, u16p, C.c_int64, u16p, C.c_int64, i32p,
                                                C.c_int32, C.c_float, C.c_double, C.c_int32,
                                                f64p]
        L.ora_attn_weights_one_head.restype = C.c_double
        L.ora_sparse_attn_one.argtypes = [u16p, u16p, C.c_int64, u16p, C.c_int64, i32p,
                                          C.c_int32, f32p, C.c_double, C.c_int32, C.c_int32,
                                          u16p]
        L.ora_sparse_attn_one.restype = C.c_int
        L.ora_rope_table.argtypes = [C.c_double, C.c_int32, C.c_int64, f32p]
        L.ora_rope_table.restype = C.c_int
        L.ora_rope_rows.argtypes = [u16p, u16p, C.c_int64, C.c_int32, C.c_int32, f32p,
                                    C.POINTER(C.c_int64), C.c_int32]
        L.ora_rope_rows.restype = C.c_int
        L.ora_candidate_blocks_one.argtypes = [f64p, C.c_int64, C.c_int32, C.c_int32, u8p]
        L.ora_candidate_blocks_one.restype = C.c_int64
        L.ora_grouped_output.argtypes = [u16p, u16p, u16p, C.c_int64, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, u16p, u16p]
        L.ora_grouped_output.restype = None
        L.ora_linear_bf16.argtypes = [u16p, u16p, C.c_int64, C.c_int32, C.c_int32, u16p]
        L.ora_linear_bf16.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(C.POINTER(ct))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


FP8_BLOCK = 32


# ---------------------------------------------------------------- scalars
def bf16_to_float(h: int) -> float:
    return lib().ora_bf16_to_double(int(h))


def float_to_bf16(x: float) -> int:
    return int(lib().ora_double_to_bf16(float(x)))


def pow2_ceil(v: float) -> float:
    return float(lib().ora_pow2_ceil(float(v)))


def e4m3_round(y: float) -> float:
    return float(lib().ora_e4m3_round(float(y)))


# ---------------------------------------------------------------- fp8
def fp8_round_rows(x: np.ndarray, block: int = FP8_BLOCK) -> np.ndarray:
    """bf16 rows [..., row_len] (uint16 bits) -> fp8-rounded bf16 rows."""
    x = _c(x, np.uint16)
    row_len = x.shape[-1]
    rows = x.size // row_len if row_len else 0
    out = np.empty_like(x)
    rc = lib().ora_fp8_round_rows(_p(x, C.c_uint16), _p(out, C.c_uint16), rows, row_len, block)
    if rc != 0:
        raise ValueError("row_len must be a multiple of the fp8 block")
    return out


# ---------------------------------------------------------------- window
def window_idx(start_pos: int, n_tokens: int, window: int) -> np.ndarray:
    cols = min(n_tokens, window) if start_pos == 0 else window
    idx = np.empty((n_tokens, cols), dtype=np.int32)
    rc = lib().ora_window_idx(start_pos, n_tokens, window, _p(idx, C.c_int32))
    if rc < 0:
        raise ValueError("a decode call (start_pos > 0) takes exactly one token")
    return idx


def causal_count(pos: int, ratio: int, n_rows: int) -> int:
    return int(lib().ora_causal_count(pos, ratio, n_rows))


class WindowCache:
    """The ring [window][row_len]: token p lives in slot p mod window."""

    def __init__(self, window: int, row_len: int):
        self.window = window
        self.rows = np.zeros((window, row_len), dtype=np.uint16)
        self.token = np.full(window, -1, dtype=np.int64)

    def prefill(self, rows: np.ndarray, start_pos: int = 0) -> None:
        T = rows.shape[0]
        for t in range(max(0, T - self.window), T):
            slot = (start_pos + t) % self.window
            self.rows[slot] = rows[t]
            self.token[slot] = start_pos + t

    def put(self, row: np.ndarray, pos: int) -> int:
        slot = pos % self.window
        self.rows[slot] = row
        self.token[slot] = pos
        return slot


# ---------------------------------------------------------------- indexer
def indexer_scores(qI: np.ndarray, kI: np.ndarray, w: np.ndarray, start_pos: int,
                   ratio: int, cand: np.ndarray | None = None, cand_block: int = 1,
                   tokens=None) -> np.ndarray:
    """qI [T, HI, DI], kI [L, DI] bf16; w [T, HI] f32; cand [T, cand_width] u8.
    Returns double scores [len(tokens), L] with -inf where excluded."""
    qI = _c(qI, np.uint16)
    kI = _c(kI, np.uint16)
    w = _c(w, np.float32)
    T, HI, DI = qI.shape
    L = kI.shape[0]
    toks = range(T) if tokens is None else tokens
    toks = list(toks)
    out = np.empty((len(toks), L), dtype=np.float64)
    cand_c = None if cand is None else _c(cand, np.uint8)
    for r, t in enumerate(toks):
        n_valid = causal_count(start_pos + t, ratio, L)
        cp = None if cand_c is None else cand_c[t].ctypes.data_as(C.POINTER(C.c_uint8))
        row = out[r]
        lib().ora_indexer_scores_one(qI[t].ctypes.data_as(C.POINTER(C.c_uint16)),
                                     _p(kI, C.c_uint16),
                                     w[t].ctypes.data_as(C.POINTER(C.c_float)), cp,
                                     cand_block, HI, DI, L, n_valid,
                                     row.ctypes.data_as(C.POINTER(C.c_double)))
    return out


# ---------------------------------------------------------------- top-k
def topk(scores: np.ndarray, k: int, offset: int = 0) -> np.ndarray:
    """scores [R, L] (any float dtype; converted exactly to double) ->
    int32 [R, k]: the selected positions + offset in ascending position order
    (the selection ranks by score desc, then position asc), -1 pad."""
    s = _c(np.asarray(scores, dtype=np.float64), np.float64)
    R, L = s.shape
    out = np.empty((R, k), dtype=np.int32)
    for r in range(R):
        m = lib().ora_topk_one(s[r].ctypes.data_as(C.POINTER(C.c_double)), L, k, offset,
                               out[r].ctypes.data_as(C.POINTER(C.c_int32)))
        if m < 0:
            raise MemoryError("oracle top-k allocation failed")
    return out


# ---------------------------------------------------------------- attention
def sparse_attn(q: np.ndarray, rows_a: np.ndarray, rows_b: np.ndarray | None,
                idx: np.ndarray, sink: np.ndarray, scale: float,
                queries=None) -> np.ndarray:
    """q [T, H, D] bf16; rows_a [A, D]; rows_b [Lb, D] or None; idx [T, width]
    int32 (window entries < A, compressed entries offset by A, -1 skipped);
    sink [H] f32.  Returns bf16 [len(queries), H, D]."""
    q = _c(q, np.uint16)
    rows_a = _c(rows_a, np.uint16)
    idx = _c(idx, np.int32)
    sink = _c(sink, np.float32)
    T, H, D = q.shape
    A = rows_a.shape[0]
    if rows_b is None:
        rb = np.zeros((1, D), dtype=np.uint16)
        Lb = 0
    else:
        rb = _c(rows_b, np.uint16)
        Lb = rb.shape[0]
    width = idx.shape[1]
    qs = list(range(T) if queries is None else queries)
    out = np.empty((len(qs), H, D), dtype=np.uint16)
    for r, t in enumerate(qs):
        rc = lib().ora_sparse_attn_one(q[t].ctypes.data_as(C.POINTER(C.c_uint16)),
                                       _p(rows_a, C.c_uint16), A, _p(rb, C.c_uint16), Lb,
                                       idx[t].ctypes.data_as(C.POINTER(C.c_int32)), width,
                                       _p(sink, C.c_float), float(scale), H, D,
                                       out[r].ctypes.data_as(C.POINTER(C.c_uint16)))
        if rc != 0:
            raise MemoryError("oracle attention allocation failed")
    return out


def attn_weights(q_h: np.ndarray, rows_a: np.ndarray, rows_b: np.ndarray | None,
                 idx_row: np.ndarray, sink_h: float, scale: float):
    """Weights A_i of one head of one query and the sink's share."""
    q_h = _c(q_h, np.uint16)
    rows_a = _c(rows_a, np.uint16)
    idx_row = _c(idx_row, np.int32)
    D = q_h.shape[0]
    if rows_b is None:
        rb = np.zeros((1, D), dtype=np.uint16)
        Lb = 0
    else:
        rb = _c(rows_b, np.uint16)
        Lb = rb.shape[0]
    wts = np.empty(idx_row.shape[0], dtype=np.float64)
    share = lib().ora_attn_weights_one_head(_p(q_h, C.c_uint16), _p(rows_a, C.c_uint16),
                                            rows_a.shape[0], _p(rb, C.c_uint16), Lb,
                                            _p(idx_row, C.c_int32), idx_row.shape[0],
                                            float(sink_h), float(scale), D,
                                            wts.ctypes.data_as(C.POINTER(C.c_double)))
    return wts, float(share)


def scores_to_f32(s: np.ndarray) -> np.ndarray:
    """Oracle scores rounded once to binary32 (the precision the scores are
    handed over in)."""
    return np.asarray(s, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- RoPE
def rope_table(theta: float, rope_dim: int, n_pos: int) -> np.ndarray:
    """f32 [n_pos, rope_dim/2, 2]: (cos, sin) of p * theta^(-2i/rope_dim),
    each rounded once to binary32 (freqs_cis at ratio 0)."""
    out = np.empty((n_pos, rope_dim // 2, 2), dtype=np.float32)
    rc = lib().ora_rope_table(float(theta), rope_dim, n_pos, _p(out, C.c_float))
    if rc != 0:
        raise ValueError("rope_dim must be even and positive, theta positive")
    return out


def rope_rows(x: np.ndarray, table: np.ndarray, row_pos, rope_dim: int,
              inverse: bool = False) -> np.ndarray:
    """bf16 rows [..., row_len] (uint16 bits): the last rope_dim values of row
    r rotated by table[row_pos[r]] (negated angle when inverse), binary32
    products, bf16 results; row_pos has one entry per row of the flattened
    leading axes."""
    x = _c(x, np.uint16)
    row_len = x.shape[-1]
    rows = x.size // row_len
    pos = _c(np.asarray(row_pos).reshape(-1), np.int64)
    if pos.shape[0] != rows:
        raise ValueError("one position per row")
    tab = _c(table, np.float32)
    if pos.size and (pos.min() < 0 or pos.max() >= tab.shape[0]):
        raise ValueError("position outside the table")
    if tab.ndim != 3 or tab.shape[1] * 2 != rope_dim or tab.shape[2] != 2:
        raise ValueError("table must be [n_pos, rope_dim/2, 2]")
    out = np.empty_like(x)
    rc = lib().ora_rope_rows(_p(x, C.c_uint16), _p(out, C.c_uint16), rows, row_len, rope_dim,
                             _p(tab, C.c_float), _p(pos, C.c_int64), 1 if inverse else 0)
    if rc != 0:
        raise ValueError("rope_dim must be even, positive and at most row_len")
    return out


def rope_fp8_rows(x: np.ndarray, table: np.ndarray, row_pos, rope_dim: int) -> np.ndarray:
    """The window-key epilogue: RoPE on the last rope_dim values (bf16 out),
    then the fp8 round trip of the whole row (W_{t,448:} <- R_t w; W <- FP8(W))."""
    return fp8_round_rows(rope_rows(x, table, row_pos, rope_dim))


# ---------------------------------------------------------------- candidate blocks
def candidate_blocks(scores: np.ndarray, cand_block: int, topk_blocks: int) -> np.ndarray:
    """scores [R, L] (converted exactly to double) -> u8 mask [R, ceil(L /
    cand_block)]: 1 for the topk_blocks blocks with the largest block score
    (the largest valid score of the block's positions), ties to the lower
    block, blocks with no valid score never chosen."""
    if cand_block < 1 or topk_blocks < 1:
        raise ValueError("cand_block and topk_blocks must be positive")
    s = _c(np.asarray(scores, dtype=np.float64), np.float64)
    R, L = s.shape
    nb = -(-L // cand_block)
    out = np.zeros((R, nb), dtype=np.uint8)
    for r in range(R):
        m = lib().ora_candidate_blocks_one(s[r].ctypes.data_as(C.POINTER(C.c_double)), L,
                                           cand_block, topk_blocks,
                                           out[r].ctypes.data_as(C.POINTER(C.c_uint8)))
        if m < 0:
            raise ValueError("cand_block and topk_blocks must be positive")
    return out


# ---------------------------------------------------------------- grouped output
def grouped_output(o_bar: np.ndarray, wo_a: np.ndarray, wo_b: np.ndarray, groups: int):
    """o_bar [T, H, D] (or [T, H*D]) bf16 after the inverse rotation; wo_a
    [groups*rank, gw]; wo_b [dim, groups*rank].  Returns (og [T, groups*rank],
    x [T, dim]) as bf16 bits: each projection a double sum rounded once."""
    o = _c(o_bar, np.uint16)
    T = o.shape[0]
    o = o.reshape(T, -1)
    wa = _c(wo_a, np.uint16)
    wb = _c(wo_b, np.uint16)
    gr, gw = wa.shape
    if gr % groups or o.shape[1] != groups * gw or wb.shape[1] != gr:
        raise ValueError("shapes do not match the grouping")
    og = np.empty((T, gr), dtype=np.uint16)
    x = np.empty((T, wb.shape[0]), dtype=np.uint16)
    lib().ora_grouped_output(_p(o, C.c_uint16), _p(wa, C.c_uint16), _p(wb, C.c_uint16), T,
                             groups, gr // groups, gw, wb.shape[0], _p(og, C.c_uint16),
                             _p(x, C.c_uint16))
    return og, x


def linear_bf16(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """a [M, K], w [N, K] bf16 -> y [M, N] bf16: double sums rounded once."""
    a = _c(a, np.uint16)
    w = _c(w, np.uint16)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("a and w disagree on K")
    y = np.empty((M, N), dtype=np.uint16)
    lib().ora_linear_bf16(_p(a, C.c_uint16), _p(w, C.c_uint16), M, N, K, _p(y, C.c_uint16))
    return y
