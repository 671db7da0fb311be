"""Thin Python binding of libv41 (the gfx950 HIP library): one function per C
entry point, with the same name and argument order.  It only marshals
arguments -- tensors become device pointers, the stream defaults to torch's
current stream -- and raises V41Error on a non-zero status.  There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libv41.so")

V41_OK, V41_EINVAL, V41_EHIP, V41_EDEVICE = 0, -1, -2, -3
EXPORTS = ("v41_last_error", "v41_abi_version", "v41_fp8_round_rows", "v41_window_idx",
           "v41_indexer_scores", "v41_topk_select", "v41_sparse_attn_sink",
           "v41_sparse_attn_workspace_bytes", "v41_sparse_attn_sink_noalloc", "v41_rope_table",
           "v41_rope_rows", "v41_rope_fp8_rows", "v41_decode_step", "v41_candidate_blocks",
           "v41_linear_bf16", "v41_linear_workspace_bytes", "v41_grouped_output",
           "v41_grouped_output_workspace_bytes", "v41_probe_hbm_read", "v41_probe_mfma")


class DecodeStepArgs(C.Structure):
    """v41_decode_step_args of include/v41.h, field for field."""
    _fields_ = [("batch", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("window", C.c_int32), ("ratio", C.c_int32), ("index_heads", C.c_int32),
                ("index_dim", C.c_int32), ("topk", C.c_int32), ("rope_dim", C.c_int32),
                ("scale", C.c_float), ("n_rows", C.c_int64), ("rope_rows", C.c_int64),
                ("ring_bs", C.c_int64), ("latent_bs", C.c_int64), ("kI_bs", C.c_int64),
                ("workspace_bytes", C.c_int64), ("pos", C.c_void_p), ("q", C.c_void_p),
                ("kv_new", C.c_void_p), ("ring", C.c_void_p), ("latent", C.c_void_p),
                ("kI", C.c_void_p), ("qI", C.c_void_p), ("w", C.c_void_p),
                ("rope_table", C.c_void_p), ("sink", C.c_void_p), ("scores", C.c_void_p),
                ("idx", C.c_void_p), ("out", C.c_void_p), ("workspace", C.c_void_p)]

    _POINTERS = ("pos", "q", "kv_new", "ring", "latent", "kI", "qI", "w", "rope_table", "sink",
                 "scores", "idx", "out", "workspace")

    @classmethod
    def make(cls, **kw) -> "DecodeStepArgs":
        """Fields by name; tensors (or ints, or None) for the pointer fields."""
        a = cls()
        for k, v in kw.items():
            if k in cls._POINTERS:
                setattr(a, k, _ptr(v))
            else:
                setattr(a, k, v)
        return a


class V41Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libv41 status {code}: {msg}")
        self.code = code


_lib = None


def load() -> C.CDLL:
    """Load libv41.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m indexer_top_sink_amd.build` (hipcc, gfx950)")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int32, C.c_float
    L.v41_last_error.restype = C.c_char_p
    L.v41_last_error.argtypes = []
    L.v41_abi_version.restype = C.c_int
    L.v41_abi_version.argtypes = []
    L.v41_fp8_round_rows.restype = C.c_int
    L.v41_fp8_round_rows.argtypes = [vp, i64, vp, i64, i64, i32, vp, i32, i64, vp]
    L.v41_window_idx.restype = C.c_int
    L.v41_window_idx.argtypes = [i64, i32, i32, i32, vp, i64, i64, C.POINTER(C.c_int32), vp]
    L.v41_indexer_scores.restype = C.c_int
    L.v41_indexer_scores.argtypes = [vp, vp, i64, vp, vp, i32, i32, i32, i32, i64, i32, i32,
                                     i32, i64, vp, i64, vp]
    L.v41_topk_select.restype = C.c_int
    L.v41_topk_select.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64, vp]
    L.v41_sparse_attn_sink.restype = C.c_int
    L.v41_sparse_attn_sink.argtypes = [vp, vp, i64, i64, vp, i64, i64, vp, i32, i64, vp, f32,
                                       i32, i32, i32, i32, vp, vp, i64, vp]
    L.v41_sparse_attn_sink_noalloc.restype = C.c_int
    L.v41_sparse_attn_sink_noalloc.argtypes = [vp, vp, i64, i64, vp, i64, i64, vp, i32, i64, vp,
                                               f32, i32, i32, i32, i32, vp, vp]
    L.v41_sparse_attn_workspace_bytes.restype = C.c_int64
    L.v41_sparse_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.v41_rope_table.restype = C.c_int
    L.v41_rope_table.argtypes = [C.c_double, i32, i64, vp, vp]
    L.v41_rope_rows.restype = C.c_int
    L.v41_rope_rows.argtypes = [vp, i64, vp, i64, i32, i32, i32, i32, i32, vp, i64, vp, i64,
                                i32, vp]
    L.v41_rope_fp8_rows.restype = C.c_int
    L.v41_rope_fp8_rows.argtypes = [vp, i64, vp, i64, i32, i32, i32, i32, vp, i64, vp, i64,
                                    vp, i32, i64, vp]
    L.v41_candidate_blocks.restype = C.c_int
    L.v41_candidate_blocks.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64, vp]
    L.v41_linear_bf16.restype = C.c_int
    L.v41_linear_bf16.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i32, i32, i32, i32,
                                  vp, i64, vp]
    L.v41_linear_workspace_bytes.restype = C.c_int64
    L.v41_linear_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.v41_grouped_output.restype = C.c_int
    L.v41_grouped_output.argtypes = [vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64,
                                     i32, vp, i64, vp, i64, vp]
    L.v41_grouped_output_workspace_bytes.restype = C.c_int64
    L.v41_grouped_output_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    L.v41_probe_hbm_read.restype = C.c_int
    L.v41_probe_hbm_read.argtypes = [vp, i64, i32, vp, vp]
    L.v41_probe_mfma.restype = C.c_int
    L.v41_probe_mfma.argtypes = [i32, i32, vp, vp]
    L.v41_decode_step.restype = C.c_int
    L.v41_decode_step.argtypes = [C.POINTER(DecodeStepArgs), vp]
    _lib = L
    return L


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != V41_OK:
        msg = load().v41_last_error()
        raise V41Error(rc, msg.decode() if msg else "")


def v41_last_error() -> str:
    m = load().v41_last_error()
    return m.decode() if m else ""


def v41_abi_version() -> int:
    return load().v41_abi_version()


def v41_fp8_round_rows(inp, in_ld, out, out_ld, rows, row_len, ring=None, ring_slots=0,
                       first_pos=0, stream=None) -> None:
    _check(load().v41_fp8_round_rows(_ptr(inp), in_ld, _ptr(out), out_ld, rows, row_len,
                                     _ptr(ring), ring_slots, first_pos, _stream(stream)))


def v41_window_idx(start_pos, n_tokens, window, batch, idx, idx_ld, idx_bs,
                   stream=None) -> int:
    cols = C.c_int32(0)
    _check(load().v41_window_idx(start_pos, n_tokens, window, batch, _ptr(idx), idx_ld, idx_bs,
                                 C.byref(cols), _stream(stream)))
    return cols.value


def v41_indexer_scores(qI, kI, kI_bs, w, cand, cand_width, cand_block, batch, n_tokens,
                       start_pos, ratio, n_heads, head_dim, n_rows, scores, scores_ld,
                       stream=None) -> None:
    _check(load().v41_indexer_scores(_ptr(qI), _ptr(kI), kI_bs, _ptr(w), _ptr(cand),
                                     cand_width, cand_block, batch, n_tokens, start_pos, ratio,
                                     n_heads, head_dim, n_rows, _ptr(scores), scores_ld,
                                     _stream(stream)))


def v41_topk_select(scores, n_sel_rows, n_cols, scores_ld, k, offset, idx, idx_ld,
                    stream=None) -> None:
    _check(load().v41_topk_select(_ptr(scores), n_sel_rows, n_cols, scores_ld, k, offset,
                                  _ptr(idx), idx_ld, _stream(stream)))


def v41_sparse_attn_sink(q, rows_a, rows_a_len, a_bs, rows_b, rows_b_len, b_bs, idx, width,
                         idx_ld, sink, scale, batch, n_tokens, n_heads, head_dim, out,
                         workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load().v41_sparse_attn_sink(_ptr(q), _ptr(rows_a), rows_a_len, a_bs, _ptr(rows_b),
                                       rows_b_len, b_bs, _ptr(idx), width, idx_ld, _ptr(sink),
                                       float(scale), batch, n_tokens, n_heads, head_dim,
                                       _ptr(out), _ptr(workspace), workspace_bytes,
                                       _stream(stream)))


def v41_sparse_attn_sink_noalloc(q, rows_a, rows_a_len, a_bs, rows_b, rows_b_len, b_bs, idx,
                                 width, idx_ld, sink, scale, batch, n_tokens, n_heads, head_dim,
                                 out, stream=None) -> None:
    _check(load().v41_sparse_attn_sink_noalloc(_ptr(q), _ptr(rows_a), rows_a_len, a_bs,
                                               _ptr(rows_b), rows_b_len, b_bs, _ptr(idx), width,
                                               idx_ld, _ptr(sink), float(scale), batch,
                                               n_tokens, n_heads, head_dim, _ptr(out),
                                               _stream(stream)))


def v41_sparse_attn_workspace_bytes(batch, n_tokens, n_heads, head_dim, width) -> int:
    return int(load().v41_sparse_attn_workspace_bytes(batch, n_tokens, n_heads, head_dim,
                                                      width))


def v41_rope_table(theta, rope_dim, n_pos, table, stream=None) -> None:
    _check(load().v41_rope_table(float(theta), rope_dim, n_pos, _ptr(table), _stream(stream)))


def v41_rope_rows(inp, in_ld, out, out_ld, batch, n_tokens, rows_per_pos, row_len, rope_dim,
                  table, table_rows, pos=None, start_pos=0, inverse=0, stream=None) -> None:
    _check(load().v41_rope_rows(_ptr(inp), in_ld, _ptr(out), out_ld, batch, n_tokens,
                                rows_per_pos, row_len, rope_dim, _ptr(table), table_rows,
                                _ptr(pos), start_pos, int(inverse), _stream(stream)))


def v41_rope_fp8_rows(inp, in_ld, out, out_ld, batch, n_tokens, row_len, rope_dim, table,
                      table_rows, pos=None, start_pos=0, ring=None, ring_slots=0, ring_bs=0,
                      stream=None) -> None:
    _check(load().v41_rope_fp8_rows(_ptr(inp), in_ld, _ptr(out), out_ld, batch, n_tokens,
                                    row_len, rope_dim, _ptr(table), table_rows, _ptr(pos),
                                    start_pos, _ptr(ring), ring_slots, ring_bs,
                                    _stream(stream)))


def v41_decode_step(args: DecodeStepArgs, stream=None) -> None:
    _check(load().v41_decode_step(C.byref(args), _stream(stream)))


def v41_candidate_blocks(scores, n_sel_rows, n_cols, scores_ld, cand_block, topk_blocks, cand,
                         cand_ld, stream=None) -> None:
    _check(load().v41_candidate_blocks(_ptr(scores), n_sel_rows, n_cols, scores_ld, cand_block,
                                       topk_blocks, _ptr(cand), cand_ld, _stream(stream)))


def v41_linear_bf16(a, lda, a_gs, w, ldw, w_gs, y, ldy, y_gs, M, N, K, groups, workspace=None,
                    workspace_bytes=0, stream=None) -> None:
    _check(load().v41_linear_bf16(_ptr(a), lda, a_gs, _ptr(w), ldw, w_gs, _ptr(y), ldy, y_gs, M,
                                  N, K, groups, _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


def v41_linear_workspace_bytes(M, N, K, groups) -> int:
    return int(load().v41_linear_workspace_bytes(M, N, K, groups))


def v41_grouped_output(o, n_tokens, n_heads, head_dim, groups, rank, dim, wo_a, wo_b, og, x,
                       rope_table=None, rope_rows=0, rope_dim=0, pos=None, start_pos=0,
                       workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load().v41_grouped_output(_ptr(o), n_tokens, n_heads, head_dim, groups, rank, dim,
                                     _ptr(wo_a), _ptr(wo_b), _ptr(og), _ptr(x), _ptr(rope_table),
                                     rope_rows, rope_dim, _ptr(pos), start_pos, _ptr(workspace),
                                     workspace_bytes, _stream(stream)))


def v41_grouped_output_workspace_bytes(n_tokens, n_heads, head_dim, groups, rank, dim) -> int:
    return int(load().v41_grouped_output_workspace_bytes(n_tokens, n_heads, head_dim, groups,
                                                         rank, dim))


def v41_probe_hbm_read(buf, nbytes, nontemporal, sink, stream=None) -> None:
    _check(load().v41_probe_hbm_read(_ptr(buf), nbytes, int(nontemporal), _ptr(sink),
                                     _stream(stream)))


def v41_probe_mfma(workgroups, iters, sink, stream=None) -> None:
    _check(load().v41_probe_mfma(workgroups, iters, _ptr(sink), _stream(stream)))
