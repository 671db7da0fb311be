"""One decode step or one prefill chunk of a layer: the five libv41 calls in
sequence on one HIP stream, with no host synchronisation in between.

decode (B sequences, one new token each at position pos):
  1. fp8 round trip of the B new kv rows, written straight into ring slot
     pos mod W of each sequence (the ring write);
  2. window indices: the whole ring, oldest first;
  3. indexer scores over the B sequences' index-key caches;
  4. top-k, written after the window columns, offset by W;
  5. sparse attention with the sink over [ring ; latent rows].
prefill (one sequence, T tokens at position 0):
  1. fp8 round trip of the chunk's kv rows into rows_a (and the last W of
     them into the ring);
  2. causal window indices into the chunk; 3.-5. as above with the offset T.
The window rows are the chunk at position 0 and the ring otherwise (the
"attn_v41.rs" AttnV41Run contract); compressed indices follow the window
columns, offset by the window row count (the join J = [J^w ; I + |W|] of the
"Compressed sparse attention" page).

With a RopeTable (the rotary epilogue before the path), q arrives before its
rotation and is rotated in place, and step 1 becomes the fused rotation + fp8
round trip + ring write of the new kv rows (W_{t,448:} <- R_t w; W <- FP8(W)).
At decode the positions are read on the device from an int32 [B] tensor.

Buffers are torch tensors owned by the caller (bf16 data as torch.bfloat16,
f32, int32, uint8).  Nothing here computes: every step is a libv41 call.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import v41

BF16 = torch.bfloat16


def to_device_bf16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
    return t.to(device).view(BF16)


def to_numpy_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class Geometry:
    n_heads: int
    head_dim: int
    window: int
    index_heads: int
    index_dim: int
    topk: int
    ratio: int
    scale: float


@dataclass
class RopeTable:
    """The ratio-0 RoPE table on the device: f32 [n_pos, rope_dim / 2, 2]."""
    table: torch.Tensor
    rope_dim: int

    @property
    def n_pos(self) -> int:
        return self.table.shape[0]


def rope_table(theta: float, rope_dim: int, n_pos: int, device, stream=None) -> RopeTable:
    t = torch.empty(n_pos, rope_dim // 2, 2, dtype=torch.float32, device=device)
    v41.v41_rope_table(theta, rope_dim, n_pos, t, stream=stream)
    return RopeTable(table=t, rope_dim=rope_dim)


@dataclass
class DecodeBuffers:
    """Device state of B sequences for one layer at decode."""
    geo: Geometry
    batch: int
    n_rows: int
    ring: torch.Tensor       # bf16 [B, W, D]
    kv_new: torch.Tensor     # bf16 [B, D]
    latent: torch.Tensor     # bf16 [B, L, D]
    kI: torch.Tensor         # bf16 [B, L, DI]
    qI: torch.Tensor         # bf16 [B, HI, DI]
    w: torch.Tensor          # f32 [B, HI]
    q: torch.Tensor          # bf16 [B, H, D]
    sink: torch.Tensor       # f32 [H]
    idx: torch.Tensor        # int32 [B, width]
    scores: torch.Tensor     # f32 [B, L]
    out: torch.Tensor        # bf16 [B, H, D]
    workspace: torch.Tensor | None

    @property
    def width(self) -> int:
        g = self.geo
        return g.window + (g.topk if g.ratio > 0 else 0)


def alloc_decode(geo: Geometry, batch: int, n_rows: int, device) -> DecodeBuffers:
    D, W, DI = geo.head_dim, geo.window, geo.index_dim
    width = W + (geo.topk if geo.ratio > 0 else 0)
    e = dict(device=device)
    ws_bytes = v41.v41_sparse_attn_workspace_bytes(batch, 1, geo.n_heads, D, width)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, **e) if ws_bytes > 0 else None
    return DecodeBuffers(
        geo=geo, batch=batch, n_rows=n_rows,
        ring=torch.zeros(batch, W, D, dtype=BF16, **e),
        kv_new=torch.zeros(batch, D, dtype=BF16, **e),
        latent=torch.zeros(batch, max(n_rows, 1), D, dtype=BF16, **e),
        kI=torch.zeros(batch, max(n_rows, 1), DI, dtype=BF16, **e),
        qI=torch.zeros(batch, geo.index_heads, DI, dtype=BF16, **e),
        w=torch.zeros(batch, geo.index_heads, dtype=torch.float32, **e),
        q=torch.zeros(batch, geo.n_heads, D, dtype=BF16, **e),
        sink=torch.zeros(geo.n_heads, dtype=torch.float32, **e),
        idx=torch.full((batch, width), -1, dtype=torch.int32, **e),
        scores=torch.zeros(batch, max(n_rows, 1), dtype=torch.float32, **e),
        out=torch.zeros(batch, geo.n_heads, D, dtype=BF16, **e),
        workspace=ws)


def decode_step(buf: DecodeBuffers, pos: int, stream=None, rope: RopeTable | None = None,
                pos_dev: torch.Tensor | None = None) -> None:
    """One decode step at position pos (the same for every sequence); with
    rope, q is rotated in place and pos_dev (int32 [B], optional) gives each
    sequence's position on the device for the rotations and the ring slot."""
    g = buf.geo
    B, D, W, L = buf.batch, g.head_dim, g.window, buf.n_rows
    width = buf.width
    slot = pos % W
    if rope is not None:
        # 0. rotate q; 1. rotate + fp8 the new rows straight into their slots
        v41.v41_rope_rows(buf.q, D, buf.q, D, B, 1, g.n_heads, D, rope.rope_dim, rope.table,
                          rope.n_pos, pos_dev, pos, 0, stream=stream)
        v41.v41_rope_fp8_rows(buf.kv_new, D, None, D, B, 1, D, rope.rope_dim, rope.table,
                              rope.n_pos, pos_dev, pos, buf.ring, W, W * D, stream=stream)
    else:
        # 1. fp8 round trip of the new rows into their ring slots
        v41.v41_fp8_round_rows(buf.kv_new, D, buf.ring.data_ptr() + 2 * slot * D, W * D, B, D,
                               stream=stream)
    # 2. the ring, oldest first
    v41.v41_window_idx(pos, 1, W, B, buf.idx, width, width, stream=stream)
    if g.ratio > 0:
        # 3. indexer scores; 4. top-k after the window columns, offset by W
        v41.v41_indexer_scores(buf.qI, buf.kI, buf.kI.shape[1] * g.index_dim, buf.w, None, 0,
                               1, B, 1, pos, g.ratio, g.index_heads, g.index_dim, L,
                               buf.scores, buf.scores.shape[1], stream=stream)
        v41.v41_topk_select(buf.scores, B, L, buf.scores.shape[1], g.topk, W,
                            buf.idx.data_ptr() + 4 * W, width, stream=stream)
    # 5. attention over [ring ; latent]
    ws_bytes = buf.workspace.numel() if buf.workspace is not None else 0
    v41.v41_sparse_attn_sink(buf.q, buf.ring, W, W * D, buf.latent if g.ratio > 0 else None,
                             L if g.ratio > 0 else 0, buf.latent.shape[1] * D, buf.idx, width,
                             width, buf.sink, g.scale, B, 1, g.n_heads, D, buf.out,
                             buf.workspace, ws_bytes, stream=stream)


def decode_step_args(buf: DecodeBuffers, pos_dev: torch.Tensor,
                     rope: RopeTable | None = None) -> "v41.DecodeStepArgs":
    """The argument block of v41_decode_step for these buffers: positions
    from the device tensor pos_dev (int32 [B]), so that a graph captured
    around the call serves every later step."""
    g = buf.geo
    D, W = g.head_dim, g.window
    return v41.DecodeStepArgs.make(
        batch=buf.batch, n_heads=g.n_heads, head_dim=D, window=W, ratio=g.ratio,
        index_heads=g.index_heads, index_dim=g.index_dim, topk=g.topk,
        rope_dim=rope.rope_dim if rope is not None else 0, scale=g.scale,
        n_rows=buf.n_rows if g.ratio > 0 else 0,
        rope_rows=rope.n_pos if rope is not None else 0,
        ring_bs=W * D, latent_bs=buf.latent.shape[1] * D, kI_bs=buf.kI.shape[1] * g.index_dim,
        workspace_bytes=buf.workspace.numel() if buf.workspace is not None else 0,
        pos=pos_dev, q=buf.q, kv_new=buf.kv_new, ring=buf.ring, latent=buf.latent, kI=buf.kI,
        qI=buf.qI, w=buf.w, rope_table=rope.table if rope is not None else None, sink=buf.sink,
        scores=buf.scores, idx=buf.idx, out=buf.out, workspace=buf.workspace)


def decode_step_fused(buf: DecodeBuffers, pos_dev: torch.Tensor, rope: RopeTable | None = None,
                      stream=None) -> None:
    """The same decode step as decode_step, as one v41_decode_step call (fewer
    launches; every position read on the device)."""
    v41.v41_decode_step(decode_step_args(buf, pos_dev, rope), stream=stream)


@dataclass
class PrefillBuffers:
    """Device state of one sequence's prefill chunk of T tokens at position 0."""
    geo: Geometry
    n_tokens: int
    n_rows: int
    kv_chunk: torch.Tensor   # bf16 [T, D] (unrounded)
    rows_a: torch.Tensor     # bf16 [T, D] (fp8-rounded chunk rows)
    ring: torch.Tensor       # bf16 [W, D]
    latent: torch.Tensor     # bf16 [L, D]
    kI: torch.Tensor         # bf16 [L, DI]
    qI: torch.Tensor         # bf16 [T, HI, DI]
    w: torch.Tensor          # f32 [T, HI]
    q: torch.Tensor          # bf16 [T, H, D]
    sink: torch.Tensor       # f32 [H]
    cand: torch.Tensor | None  # u8 [T, cand_width]
    cand_block: int
    idx: torch.Tensor        # int32 [T, width]
    scores: torch.Tensor     # f32 [T, L]
    out: torch.Tensor        # bf16 [T, H, D]

    @property
    def cols(self) -> int:
        return min(self.n_tokens, self.geo.window)

    @property
    def width(self) -> int:
        return self.cols + (self.geo.topk if self.geo.ratio > 0 else 0)


def alloc_prefill(geo: Geometry, n_tokens: int, n_rows: int, cand_width: int, cand_block: int,
                  device) -> PrefillBuffers:
    T, D, W, DI = n_tokens, geo.head_dim, geo.window, geo.index_dim
    width = min(T, W) + (geo.topk if geo.ratio > 0 else 0)
    e = dict(device=device)
    return PrefillBuffers(
        geo=geo, n_tokens=T, n_rows=n_rows,
        kv_chunk=torch.zeros(T, D, dtype=BF16, **e),
        rows_a=torch.zeros(T, D, dtype=BF16, **e),
        ring=torch.zeros(W, D, dtype=BF16, **e),
        latent=torch.zeros(max(n_rows, 1), D, dtype=BF16, **e),
        kI=torch.zeros(max(n_rows, 1), DI, dtype=BF16, **e),
        qI=torch.zeros(T, geo.index_heads, DI, dtype=BF16, **e),
        w=torch.zeros(T, geo.index_heads, dtype=torch.float32, **e),
        q=torch.zeros(T, geo.n_heads, D, dtype=BF16, **e),
        sink=torch.zeros(geo.n_heads, dtype=torch.float32, **e),
        cand=(torch.zeros(T, cand_width, dtype=torch.uint8, **e) if cand_width > 0 else None),
        cand_block=max(cand_block, 1),
        idx=torch.full((T, width), -1, dtype=torch.int32, **e),
        scores=torch.zeros(T, max(n_rows, 1), dtype=torch.float32, **e),
        out=torch.zeros(T, geo.n_heads, D, dtype=BF16, **e))


def prefill_chunk(buf: PrefillBuffers, stream=None, rope: RopeTable | None = None) -> None:
    g = buf.geo
    T, D, W, L = buf.n_tokens, g.head_dim, g.window, buf.n_rows
    width, cols = buf.width, buf.cols
    if rope is not None:
        # 0. rotate q; 1. rotate + fp8 the chunk's rows, seeding the ring
        v41.v41_rope_rows(buf.q, D, buf.q, D, 1, T, g.n_heads, D, rope.rope_dim, rope.table,
                          rope.n_pos, None, 0, 0, stream=stream)
        v41.v41_rope_fp8_rows(buf.kv_chunk, D, buf.rows_a, D, 1, T, D, rope.rope_dim,
                              rope.table, rope.n_pos, None, 0, buf.ring, W, 0, stream=stream)
    else:
        # 1. fp8 round trip of the chunk's rows, seeding the ring with the last W
        v41.v41_fp8_round_rows(buf.kv_chunk, D, buf.rows_a, D, T, D, buf.ring, W, 0,
                               stream=stream)
    # 2. causal window into the chunk
    v41.v41_window_idx(0, T, W, 1, buf.idx, width, T * width, stream=stream)
    if g.ratio > 0:
        cw = buf.cand.shape[1] if buf.cand is not None else 0
        v41.v41_indexer_scores(buf.qI, buf.kI, L * g.index_dim, buf.w, buf.cand, cw,
                               buf.cand_block, 1, T, 0, g.ratio, g.index_heads, g.index_dim, L,
                               buf.scores, buf.scores.shape[1], stream=stream)
        v41.v41_topk_select(buf.scores, T, L, buf.scores.shape[1], g.topk, T,
                            buf.idx.data_ptr() + 4 * cols, width, stream=stream)
    v41.v41_sparse_attn_sink(buf.q, buf.rows_a, T, T * D, buf.latent if g.ratio > 0 else None,
                             L if g.ratio > 0 else 0, L * D, buf.idx, width, width, buf.sink,
                             g.scale, 1, T, g.n_heads, D, buf.out, None, 0, stream=stream)
