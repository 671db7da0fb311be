"""Benchmark of the compressed-sparse-attention hot path on one MI355X.

A step is one pass of the whole path (fp8 round trip + ring write, window
indices, indexer scores, top-k, sparse attention with the sink) over one batch
of synthetic input already resident in HBM.  The default workload is the
batched decode: 64 sequences at context 32768 (8192 compressed rows each),
64 heads x 512, window 128, indexer 64 x 128, top-512; a step decodes one
token per sequence.  The prefill chunk (2048 tokens at position 0), the
long-context decode (16 sequences at context 131072 with planted ties) and one
sequence at context 4096 (latency) are reported alongside.

A decode step is one v41_decode_step call (three or four launches, positions
read on the device); the same step as the five separate calls is timed
alongside (--separate-calls makes that form the headline).

Timing.  Every input tensor exists in several copies (input sets); step i
runs on set i mod n, so a set's data was last touched n - 1 steps earlier
(for the decode workloads more than the 256 MB last-level cache in between).
One HIP graph holds one step per set and is replayed, with an event after
each replay: the value is K over the first-to-last event time, and the
replays give the median and 90th percentile of the per-step time.  Exactly
W untimed warm-up steps come first (256 by default and for the secondary
lines: the GPU raises its clocks over tens of milliseconds of sustained
work).  Per
kernel: each rep reads a 1 GiB buffer that evicts the last-level cache, then
launches the kernel once on each input set, directly, between two events, so
every launch reads its data from HBM; mean, p50 and p90 over the reps of the
per-launch time (20 untimed launches first, 100 reps).  Rooflines use the mean.
Fractions are given against the published peaks and against ceilings measured
in the same run (the library's HBM read and matrix-core probes; a 2 GiB device
copy and an 8192^3 bf16 torch.mm are reported beside them).

The CPU baseline is the oracle (plain C), run before the GPU is touched: one
thread on a bounded sample, and a process pool over the step's sequences
(tokens) on the host cores available (at most 16), with the core count and
CPU model; the prefill and decode16 lines carry the same two legs.  The
single-thread leg's oracle results also serve the `parity` entry of each
line: the GPU step's selected rows and attention output on the same inputs,
in bf16 ulp of the oracle's.

--step-only times the graph-replayed steps alone (for a kernel trace of the
step as it runs); --output-side times the output projections.

With --rope the step starts from q and kv rows before their rotation: q is
rotated in place and the fp8 call becomes the fused rotation + fp8 + ring write
(the rotary epilogue); without it that variant is reported as a secondary line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode64] [--rope]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from inputs import workloads as WL  # noqa: E402

METRIC = "decode tokens/s + prefill tokens/s per layer; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- staging
def geometry(wl):
    from indexer_top_sink_amd.layer import Geometry
    return Geometry(n_heads=wl.n_heads, head_dim=wl.head_dim, window=wl.window,
                    index_heads=wl.index_heads, index_dim=wl.index_dim, topk=wl.topk,
                    ratio=wl.ratio, scale=wl.scale)


def stage_decode(wl, device, keep_host=False):
    """Device buffers of a decode workload with its inputs uploaded; the ring
    rows are rounded through fp8 on the GPU (they were written by earlier
    steps).  Returns (buffers, host inputs or None)."""
    import torch

    from indexer_top_sink_amd import layer as LY
    from indexer_top_sink_amd import v41
    buf = LY.alloc_decode(geometry(wl), wl.batch, wl.n_rows, device)
    host = [] if keep_host else None
    for b in range(wl.batch):
        d = WL.decode_sequence(wl, b)
        buf.ring[b].copy_(LY.to_device_bf16(d["ring_raw"], device))
        buf.kv_new[b].copy_(LY.to_device_bf16(d["kv_new"][0], device))
        buf.latent[b].copy_(LY.to_device_bf16(d["latent"], device))
        buf.kI[b].copy_(LY.to_device_bf16(d["kI"], device))
        buf.qI[b].copy_(LY.to_device_bf16(d["qI"][0], device))
        buf.w[b].copy_(torch.from_numpy(d["w"][0]).to(device))
        buf.q[b].copy_(LY.to_device_bf16(d["q"][0], device))
        if keep_host:
            host.append(d)
    buf.sink.copy_(torch.from_numpy(WL.layer_sink(wl)).to(device))
    D = wl.head_dim
    v41.v41_fp8_round_rows(buf.ring, D, buf.ring, D, wl.batch * wl.window, D)
    torch.cuda.synchronize()
    return buf, host


def stage_prefill(wl, device, keep_host=False):
    import torch

    from indexer_top_sink_amd import layer as LY
    d = WL.prefill_inputs(wl)
    buf = LY.alloc_prefill(geometry(wl), wl.n_tokens, wl.n_rows, wl.cand_width,
                           wl.cand_block, device)
    buf.kv_chunk.copy_(LY.to_device_bf16(d["kv_chunk"], device))
    buf.latent.copy_(LY.to_device_bf16(d["latent"], device))
    buf.kI.copy_(LY.to_device_bf16(d["kI"], device))
    buf.qI.copy_(LY.to_device_bf16(d["qI"], device))
    buf.w.copy_(torch.from_numpy(d["w"]).to(device))
    buf.q.copy_(LY.to_device_bf16(d["q"], device))
    buf.cand.copy_(torch.from_numpy(d["cand"]).to(device))
    buf.sink.copy_(torch.from_numpy(WL.layer_sink(wl)).to(device))
    torch.cuda.synchronize()
    return buf, (d if keep_host else None)


def attach_rope(buf, wl, device):
    """The rotary epilogue's state: the ratio-0 table over every position the
    step touches, built on the GPU, and (decode) the positions as a device
    int32 [B] tensor, read on the device by the rotations and the ring write."""
    import torch

    from indexer_top_sink_amd import layer as LY
    n_pos = wl.start_pos + wl.n_tokens
    buf.rope = LY.rope_table(wl.rope_theta, wl.rope_dim, n_pos, device)
    if wl.mode == "decode":
        buf.pos_dev = torch.full((wl.batch,), wl.start_pos, dtype=torch.int32, device=device)
    torch.cuda.synchronize()


def clone_buffers(buf):
    """Another copy of every tensor of a buffer set (same values)."""
    import copy

    import torch
    new = copy.copy(buf)
    for k, v in vars(buf).items():
        if isinstance(v, torch.Tensor):
            setattr(new, k, v.clone())
    return new


# ----------------------------------------------------------------- the steps
def step_calls(buf, mode, rope=False):
    """The five calls of one step as separate closures (kernel order).  With
    rope, q is rotated in place first and the fp8 call becomes the fused
    rotation + fp8 + ring write of the kv rows."""
    from indexer_top_sink_amd import v41
    g = buf.geo
    D, W = g.head_dim, g.window
    if mode == "decode":
        B, L, width, pos = buf.batch, buf.n_rows, buf.width, buf.pos
        slot = pos % W
        ws_bytes = buf.workspace.numel() if buf.workspace is not None else 0
        if rope:
            rt = buf.rope
            first = [
                ("rope_rows", lambda: v41.v41_rope_rows(
                    buf.q, D, buf.q, D, B, 1, g.n_heads, D, rt.rope_dim, rt.table, rt.n_pos,
                    buf.pos_dev, pos, 0)),
                ("rope_fp8_rows", lambda: v41.v41_rope_fp8_rows(
                    buf.kv_new, D, None, D, B, 1, D, rt.rope_dim, rt.table, rt.n_pos,
                    buf.pos_dev, pos, buf.ring, W, W * D)),
            ]
        else:
            first = [("fp8_round_rows", lambda: v41.v41_fp8_round_rows(
                buf.kv_new, D, buf.ring.data_ptr() + 2 * slot * D, W * D, B, D))]
        return first + [
            ("window_idx", lambda: v41.v41_window_idx(pos, 1, W, B, buf.idx, width, width)),
            ("indexer_scores", lambda: v41.v41_indexer_scores(
                buf.qI, buf.kI, L * g.index_dim, buf.w, None, 0, 1, B, 1, pos, g.ratio,
                g.index_heads, g.index_dim, L, buf.scores, L)),
            ("topk_select", lambda: v41.v41_topk_select(
                buf.scores, B, L, L, g.topk, W, buf.idx.data_ptr() + 4 * W, width)),
            ("sparse_attn_sink", lambda: v41.v41_sparse_attn_sink(
                buf.q, buf.ring, W, W * D, buf.latent, L, L * D, buf.idx, width, width,
                buf.sink, g.scale, B, 1, g.n_heads, D, buf.out, buf.workspace, ws_bytes)),
        ]
    T, L, width, cols = buf.n_tokens, buf.n_rows, buf.width, buf.cols
    cw = buf.cand.shape[1] if buf.cand is not None else 0
    if rope:
        rt = buf.rope
        first = [
            ("rope_rows", lambda: v41.v41_rope_rows(
                buf.q, D, buf.q, D, 1, T, g.n_heads, D, rt.rope_dim, rt.table, rt.n_pos, None,
                0, 0)),
            ("rope_fp8_rows", lambda: v41.v41_rope_fp8_rows(
                buf.kv_chunk, D, buf.rows_a, D, 1, T, D, rt.rope_dim, rt.table, rt.n_pos, None,
                0, buf.ring, W, 0)),
        ]
    else:
        first = [("fp8_round_rows", lambda: v41.v41_fp8_round_rows(
            buf.kv_chunk, D, buf.rows_a, D, T, D, buf.ring, W, 0))]
    return first + [
        ("window_idx", lambda: v41.v41_window_idx(0, T, W, 1, buf.idx, width, T * width)),
        ("indexer_scores", lambda: v41.v41_indexer_scores(
            buf.qI, buf.kI, L * g.index_dim, buf.w, buf.cand, cw, buf.cand_block, 1, T, 0,
            g.ratio, g.index_heads, g.index_dim, L, buf.scores, L)),
        ("topk_select", lambda: v41.v41_topk_select(
            buf.scores, T, L, L, g.topk, T, buf.idx.data_ptr() + 4 * cols, width)),
        ("sparse_attn_sink", lambda: v41.v41_sparse_attn_sink(
            buf.q, buf.rows_a, T, T * D, buf.latent, L, L * D, buf.idx, width, width, buf.sink,
            g.scale, 1, T, g.n_heads, D, buf.out, None, 0)),
    ]


def capture(fns, torch):
    """One HIP graph replaying fns in order on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:      # warm the launch path before capture
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_replays(graphs, reps, torch):
    """Mean ms per replay over `reps` replays cycling through `graphs`."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def stats(xs):
    """mean, median and 90th percentile of a list of times."""
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


class CacheEvictor:
    """Reads a 1 GiB buffer (four times the 256 MB last-level cache): after it
    the cache holds only clean lines of this buffer, so the next kernel's
    data comes from HBM and no dirty line of earlier work is written back
    inside the timed region.  It also keeps the GPU busy long enough for the
    host to queue the timed launches behind it."""

    def __init__(self, torch, device, mib=1024):
        self.buf = torch.ones(mib << 18, dtype=torch.float32, device=device)
        self.sink = torch.empty((), dtype=torch.float32, device=device)

    def __call__(self, torch):
        torch.sum(self.buf, dim=0, out=self.sink)


KERNEL_WARMUP = 20   # untimed launches of each kernel first
KERNEL_REPS = 100    # timed reps, each after an eviction


def time_kernel(fns, reps, evict, torch):
    """Per-launch ms of one kernel: fns launch it once on each input set.
    KERNEL_WARMUP untimed launches first (cycling over the sets); then every
    rep evicts the last-level cache and launches fns directly (no graph: the
    launches queue up behind the eviction, so they run back to back) between
    two events; returns mean, p50 and p90 over the reps of the per-launch
    average."""
    st = torch.cuda.current_stream()
    for i in range(max(KERNEL_WARMUP, len(fns))):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        evict(torch)
        e0.record(st)
        for f in fns:
            f()
        e1.record(st)
    torch.cuda.synchronize()
    return stats([e0.elapsed_time(e1) / len(fns) for e0, e1 in ev])


def measured_ceilings(torch, device):
    """What this GPU reaches on plain work, for fractions beside the
    published peaks (best of 5 each):
      hbm_GBs        the library's read probe over 2 GiB, non-temporal loads
                     (the decode kernels mostly read);
      hbm_copy_GBs   a 2 GiB torch device copy, bytes read + written;
      mfma_bf16_TFLOPs  the library's matrix-core probe: independent
                     v_mfma_f32_16x16x32_bf16 chains on registers, 512
                     workgroups of four wavefronts, a 0.3 ms burst (and a
                     1.7 ms run: mfma_bf16_sustained_TFLOPs);
      gemm_bf16_TFLOPs  an 8192^3 bf16 torch.mm (a library GEMM)."""
    from indexer_top_sink_amd import v41
    n = 2 << 30
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        t = 1e30
        for _ in range(5):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t = min(t, e0.elapsed_time(e1))
        return t

    src = torch.ones(n // 4, dtype=torch.float32, device=device)
    sink = torch.zeros(4, dtype=torch.int32, device=device)
    t_read = best(lambda: v41.v41_probe_hbm_read(src, n, 1, sink))
    t_read_c = best(lambda: v41.v41_probe_hbm_read(src, n, 0, sink))
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    del src, dst
    wgs = 512
    fsink = torch.zeros(4, dtype=torch.float32, device=device)
    # a burst of about 0.3 ms (the length of a few layers' kernels) and a run
    # of about 1.7 ms, over which the clock settles lower
    t_mfma = best(lambda: v41.v41_probe_mfma(wgs, 1500, fsink))
    t_mfma_long = best(lambda: v41.v41_probe_mfma(wgs, 8000, fsink))
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device=device)
    b = torch.randn(m, m, dtype=torch.bfloat16, device=device)
    c = torch.empty(m, m, dtype=torch.bfloat16, device=device)
    t_mm = best(lambda: torch.mm(a, b, out=c))
    del a, b, c
    torch.cuda.synchronize()
    return {"hbm_GBs": round(n / (t_read * 1e-3) / 1e9, 1),
            "hbm_cached_loads_GBs": round(n / (t_read_c * 1e-3) / 1e9, 1),
            "hbm_copy_GBs": round(2 * n / (t_copy * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(524288 * wgs * 1500 / (t_mfma * 1e-3) / 1e12, 1),
            "mfma_bf16_sustained_TFLOPs": round(524288 * wgs * 8000 / (t_mfma_long * 1e-3) / 1e12,
                                                1),
            "gemm_bf16_TFLOPs": round(2 * m ** 3 / (t_mm * 1e-3) / 1e12, 1),
            "how": "hbm: v41_probe_hbm_read over 2 GiB (non-temporal, and default loads); "
                   "copy: 2 GiB torch copy (read + write bytes); mfma: v41_probe_mfma "
                   "(512 x 4 wavefronts x 1500 (sustained: 8000) x 8 independent 16x16x32 "
                   "bf16); gemm: 8192^3 "
                   "bf16 torch.mm; best of 5 each"}


# ----------------------------------------------------------------- algorithmic work
def algorithmic(wl, host_idx=None, valid_pairs=None, rope=False):
    """Bytes and flops per kernel of one step (what the method must move or
    compute).  Attention flops count 4 * H * D per valid index entry; indexer
    flops 2 * HI * DI per visible (query, position) pair.  The rotary
    epilogue moves the rotated tail of every q head in place, one table row
    per position, and the kv rows in and out (plus the ring copy)."""
    H, D, HI, DI, W = wl.n_heads, wl.head_dim, wl.index_heads, wl.index_dim, wl.window
    Q, L = wl.queries, wl.n_rows
    if wl.mode == "decode":
        pairs = Q * L if valid_pairs is None else valid_pairs
        idx_valid = Q * wl.width if host_idx is None else int((host_idx >= 0).sum())
        fp8_rows = Q
    else:
        pairs = valid_pairs
        idx_valid = int((host_idx >= 0).sum())
        fp8_rows = wl.n_tokens
    k = {}
    k["fp8_round_rows"] = {"bytes": fp8_rows * D * 2 * 2, "flops": 0}
    k["window_idx"] = {"bytes": Q * wl.window_cols * 4, "flops": 0}
    k["indexer_scores"] = {"bytes": pairs * DI * 2 + Q * HI * DI * 2 + Q * HI * 4 + Q * L * 4,
                           "flops": pairs * 2 * HI * DI}
    if wl.mode == "prefill":
        # the index keys are read once per chunk; each visible pair reuses them
        k["indexer_scores"]["bytes"] = L * DI * 2 + Q * HI * DI * 2 + Q * HI * 4 + Q * L * 4 + \
            Q * wl.cand_width
    k["topk_select"] = {"bytes": Q * L * 4 + Q * wl.topk * 4, "flops": 0}
    rows_bytes = idx_valid * D * 2
    if wl.mode == "prefill":
        rows_bytes = (wl.n_tokens + L) * D * 2   # every row source read once
    k["sparse_attn_sink"] = {"bytes": rows_bytes + Q * wl.width * 4 + 2 * Q * H * D * 2,
                             "flops": idx_valid * 4 * H * D}
    if rope:
        rd = wl.rope_dim
        table = Q * rd // 2 * 8      # one table row per distinct position
        del k["fp8_round_rows"]
        k["rope_rows"] = {"bytes": Q * H * rd * 2 * 2 + table, "flops": 0}
        ring_rows = min(wl.n_tokens, wl.window) * wl.batch
        kv_out = fp8_rows if wl.mode == "prefill" else 0   # decode writes the ring only
        k["rope_fp8_rows"] = {"bytes": fp8_rows * D * 2 + (kv_out + ring_rows) * D * 2 + table,
                              "flops": 0}
    return k


def time_candidate_blocks(torch, device, steps):
    """The candidate-source selection at decode16's shape: 16 score rows of
    32768 positions, the best 2048 of 4096 blocks of 8.  Per-launch us and the
    algorithmic bytes (scores read once, one mask byte per block written)."""
    from inputs import synth
    from indexer_top_sink_amd import v41
    R, L, cb, kb = 16, 32768, 8, 2048
    s = torch.from_numpy(synth.normal_f32(0x5EED4999, synth.TAG_MISC, (R, L))).to(device)
    cand = torch.empty(R, L // cb, dtype=torch.uint8, device=device)
    fn = lambda: v41.v41_candidate_blocks(s, R, L, L, cb, kb, cand, L // cb)
    g = capture([fn] * 8, torch)
    us = time_replays([g], max(4, steps // 8), torch) * 1e3 / 8
    nbytes = R * L * 4 + R * (L // cb)
    return {"shape": f"{R} rows x {L} positions, top {kb} of {L // cb} blocks of {cb}",
            "avg_us": round(us, 2), "algorithmic_bytes": nbytes,
            "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def time_grouped_output(torch, device, steps, n_tokens):
    """The output side of a step: the inverse rotation of o's tails (in
    place), wo_a (8 groups, rank 1024, 4096 features each) and wo_b
    (5120 x 8192), synthetic N(0, 1/fan_in) bf16 weights.  Per-step us, the
    projections alone, the weight stream (decode) and the MFMA rate (prefill)
    of the projections."""
    from inputs import synth
    from indexer_top_sink_amd import layer as LY
    from indexer_top_sink_amd import v41
    T, H, D, G, R, dim, rd = n_tokens, 64, 512, 8, 1024, 5120, 64
    gw = H * D // G

    def weights(seed, shape, fan_in):
        x = synth.normal_f32(seed, synth.TAG_MISC, shape) * (1.0 / fan_in ** 0.5)
        return LY.to_device_bf16(synth.f32_to_bf16_bits(x), device)

    wa, wb = weights(0x5EED5001, (G * R, gw), gw), weights(0x5EED5002, (dim, G * R), G * R)
    o = LY.to_device_bf16(synth.normal_bf16(0x5EED5003, synth.TAG_Q, (T, H, D)), device)
    pos = 32767 if T <= 64 else 0
    rt = LY.rope_table(10000.0, rd, pos + T, device)
    og = torch.empty(T, G * R, dtype=torch.bfloat16, device=device)
    x = torch.empty(T, dim, dtype=torch.bfloat16, device=device)
    wsb = v41.v41_grouped_output_workspace_bytes(T, H, D, G, R, dim)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=device)
    # o before its inverse rotation, which the call applies in place (token t
    # at position pos + t for a chunk, pos for every decode sequence); o keeps
    # turning back across replays, which changes no cost
    posd = torch.full((T,), pos, dtype=torch.int32, device=device)
    step = lambda: v41.v41_grouped_output(
        o, T, H, D, G, R, dim, wa, wb, og, x, rope_table=rt.table, rope_rows=rt.n_pos,
        rope_dim=rd, pos=posd if T <= 64 else None, start_pos=pos, workspace=ws,
        workspace_bytes=wsb)
    proj = lambda: v41.v41_grouped_output(o, T, H, D, G, R, dim, wa, wb, og, x, workspace=ws,
                                          workspace_bytes=wsb)
    reps = max(4, steps // 4)
    g_all = capture([step] * 4, torch)
    us_all = time_replays([g_all], reps, torch) * 1e3 / 4
    g_proj = capture([proj] * 4, torch)
    us_proj = time_replays([g_proj], reps, torch) * 1e3 / 4
    wbytes = (G * R * gw + dim * G * R) * 2
    flops = 2 * T * (G * R * gw + dim * G * R)
    return {"tokens": T, "us_per_step": round(us_all, 2), "projections_us": round(us_proj, 2),
            "weight_bytes": wbytes, "weights_GBs": round(wbytes / (us_proj * 1e-6) / 1e9, 1),
            "flops": flops, "TFLOPs": round(flops / (us_proj * 1e-6) / 1e12, 1)}


# ----------------------------------------------------------------- CPU baseline
def _oracle_decode(job):
    """Worker: the oracle's decode step for each listed sequence; returns
    (sequences done, seconds inside the oracle, {sequence: (idx, out)} when
    asked to keep the outputs)."""
    import oracle as O
    from oracle import layer as OL
    name, seqs, keep = job
    wl = WL.WORKLOADS[name]
    sink = WL.layer_sink(wl)
    busy = 0.0
    outs = {}
    for b in seqs:
        d = WL.decode_sequence(wl, b)
        ring = O.WindowCache(wl.window, wl.head_dim)
        ring.rows[:] = O.fp8_round_rows(d["ring_raw"])
        t0 = time.perf_counter()
        res = OL.decode(ring, d["kv_new"], wl.start_pos, d["q"], sink, wl.scale, ratio=wl.ratio,
                        latent=d["latent"], kI=d["kI"], qI=d["qI"], w=d["w"], k=wl.topk)
        busy += time.perf_counter() - t0
        if keep:
            outs[b] = (res["idx"][0], res["out"][0])
    return len(seqs), busy, outs


def _oracle_prefill(job):
    """Worker: the oracle's prefill chunk over the listed tokens (and, when
    asked, their idx rows and outputs)."""
    from oracle import layer as OL
    name, toks, keep = job
    wl = WL.WORKLOADS[name]
    d = WL.prefill_inputs(wl)
    t0 = time.perf_counter()
    res = OL.prefill(d["kv_chunk"], d["q"], WL.layer_sink(wl), wl.scale, wl.window,
                     ratio=wl.ratio, latent=d["latent"], kI=d["kI"], qI=d["qI"], w=d["w"],
                     cand=d["cand"], cand_block=wl.cand_block, k=wl.topk, queries=list(toks))
    t = time.perf_counter() - t0
    outs = {t_: (res["idx"][i], res["out"][i]) for i, t_ in enumerate(toks)} if keep else {}
    return len(toks), t, outs


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count() or 1, avail


def cpu_baseline(wl, budget_s=10.0, max_workers=16):
    """The oracle (plain C, double precision), as it stands, on the host cores,
    two ways: one thread on the first sequences (tokens) of the workload until
    about budget_s of oracle time, and a process pool over independent
    sequences (tokens), one worker per available core up to max_workers (the
    host share of one GPU), whose throughput is the work done over the
    busiest worker's oracle time.  Runs before this process touches the GPU,
    so the pool's fork is safe."""
    import multiprocessing as mp
    model, nproc, avail = host_cpu()
    workers = max(1, min(max_workers, avail))
    outputs = {}  # the single-thread leg's oracle results, for the parity report
    if wl.mode == "decode":
        done, busy = 0, 0.0
        while done < wl.batch and busy < budget_s:
            n, t, o = _oracle_decode((wl.name, [done], True))
            done += n
            busy += t
            outputs.update(o)
        single = {"value": done / busy, "seconds": round(busy, 3),
                  "sample": f"{done} of {wl.batch} sequences, one decode step each"}
        chunks = [list(range(wl.batch))[i::workers] for i in range(workers)]
        jobs = [(wl.name, c, False) for c in chunks if c]
        fn = _oracle_decode
        unit_name = "sequences"
    else:
        toks = list(range(wl.n_tokens - 16, wl.n_tokens))    # the costliest tokens
        n, t, outputs = _oracle_prefill((wl.name, toks, True))
        single = {"value": n / t, "seconds": round(t, 3),
                  "sample": f"the last {n} of {wl.n_tokens} prefill tokens (the longest rows)"}
        span = list(range(wl.n_tokens - 16 * workers, wl.n_tokens))
        jobs = [(wl.name, span[i::workers], False) for i in range(workers)]
        fn = _oracle_prefill
        unit_name = "tokens"
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        res = pool.map(fn, jobs)
    wall = time.perf_counter() - t0
    n_all = sum(r[0] for r in res)
    busiest = max(r[1] for r in res)
    return {"value": round(n_all / busiest, 3), "unit": "tokens/s", "cores": len(jobs),
            "_outputs": outputs,
            "kind": "oracle",
            "sample": f"{n_all} {unit_name} of one step over {len(jobs)} worker processes "
                      f"(throughput = work / busiest worker's oracle seconds)",
            "seconds": round(busiest, 3), "pool_wall_s": round(wall, 3),
            "single_thread": {**{k: (round(v, 3) if isinstance(v, float) else v)
                                 for k, v in single.items()}, "unit": "tokens/s",
                              "cores": 1},
            "cpu_model": model, "nproc": nproc, "cores_available": avail}


# ------------------------------------------------------------- parity
ATTN_ULPS, ATTN_ATOL = 2.0, 1e-2   # the attention parity criterion of the tests


def _bf16_f64(bits):
    w = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return w.view(np.float32).astype(np.float64)


def parity_report(buf, wl, oracle_outputs):
    """GPU results of input set 0 against the oracle results that the CPU leg
    kept (its single-thread sample): the selected rows (window part exactly,
    the top-k part as a set) and, where both sides selected the same rows,
    the attention output in bf16 ulp of the oracle's value (pass: within 2
    ulp or 1e-2 absolute)."""
    from indexer_top_sink_amd import layer as LY
    if not oracle_outputs:
        return None
    keys = sorted(oracle_outputs)
    idx = buf.idx.cpu().numpy()
    out = LY.to_numpy_bf16(buf.out)
    W = idx.shape[1] - wl.topk
    same, errs_ulp, errs_abs = 0, [], []
    for r in keys:
        o_idx, o_out = oracle_outputs[r]
        if not (np.array_equal(idx[r, :W], o_idx[:W]) and
                np.array_equal(np.sort(idx[r, W:]), np.sort(o_idx[W:]))):
            continue
        same += 1
        g, o = _bf16_f64(out[r]), _bf16_f64(o_out)
        err = np.abs(g - o)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o), 2.0 ** -126))) - 7)
        errs_ulp.append((err / ulp).ravel())
        errs_abs.append(err.ravel())
    unit = "sequences" if wl.mode == "decode" else "tokens"
    rep = {"sample": f"{len(keys)} {unit} ({unit[:-1]} {keys[0]}..{keys[-1]}), the CPU leg's "
                     "oracle outputs against the GPU step on the same inputs",
           "selection_equal": f"{same} of {len(keys)}"}
    if errs_ulp:
        u, a = np.concatenate(errs_ulp), np.concatenate(errs_abs)
        rep.update({"outputs": int(u.size), "max_ulp": round(float(u.max()), 2),
                    "frac_within_2ulp": round(float((u <= ATTN_ULPS).mean()), 6),
                    "max_abs": float(a.max()),
                    "fail": int(((u > ATTN_ULPS) & (a > ATTN_ATOL)).sum())})
    return rep


# ----------------------------------------------------------------- main
def timed_steps(step_fns, steps, warmup, torch):
    """K steps: replays of one HIP graph that holds one step per input set
    (n steps per replay, as one graph would hold a model's layers), with an
    event after each replay, plus single-step graphs for a remainder of K.
    Returns the mean ms per step over all K (first event to last), the
    mean/p50/p90 over the full replays of the per-step time, and the
    single-step graphs.  Exactly W warm-up steps first."""
    n = len(step_fns)
    all_graph = capture([f for c in step_fns for f in c], torch)
    one_graphs = [capture(c, torch) for c in step_fns]
    # exactly W warm-up steps: full replays, then single steps
    w_full, w_rest = divmod(warmup, n)
    for _ in range(w_full):
        all_graph.replay()
    for i in range(w_rest):
        one_graphs[i].replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    full, rest = divmod(steps, n)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(full + 2)]
    ev[0].record(st)
    for i in range(full):
        all_graph.replay()
        ev[i + 1].record(st)
    for i in range(rest):
        one_graphs[i].replay()
    ev[-1].record(st)
    ev[-1].synchronize()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) / n for i in range(full)] or \
        [ev[0].elapsed_time(ev[-1]) / steps]
    return ev[0].elapsed_time(ev[-1]) / steps, stats(per), one_graphs


def fused_call(buf, rope):
    """The whole decode step as one v41_decode_step call (device positions)."""
    from indexer_top_sink_amd import layer as LY
    from indexer_top_sink_amd import v41
    args = LY.decode_step_args(buf, buf.pos_dev, buf.rope if rope else None)
    return lambda: v41.v41_decode_step(args)


# Warm-up steps of the secondary lines: enough to carry the GPU past its
# clock ramp (tens of milliseconds of work; the headline takes W from the
# command line)
SECONDARY_WARMUP = 256


def run_workload(name, steps, warmup, n_sets, torch, device, evict, rope=False,
                 separate=False, oracle_outputs=None):
    """Times K steps of a workload.  A decode step is one v41_decode_step call
    (unless separate); its separate-call form is timed alongside.  Per-kernel
    times: each kernel launched once on each input set in one graph, every
    replay after a cache eviction.  Returns a dict."""
    wl = WL.WORKLOADS[name]
    t0 = time.time()
    if wl.mode == "decode":
        buf0, _ = stage_decode(wl, device)
        buf0.pos = wl.start_pos
        buf0.pos_dev = torch.full((wl.batch,), wl.start_pos, dtype=torch.int32, device=device)
    else:
        buf0, _ = stage_prefill(wl, device)
    if rope:
        attach_rope(buf0, wl, device)
    sets = [buf0] + [clone_buffers(buf0) for _ in range(n_sets - 1)]
    for s in sets:
        s.pos = getattr(buf0, "pos", 0)
    log(f"{name}: staged {n_sets} input sets in {time.time() - t0:.1f}s")

    calls = [step_calls(s, wl.mode, rope) for s in sets]
    sep_fns = [[f for _, f in c] for c in calls]
    ms_sep = sep_stats = None
    if wl.mode == "decode" and not separate:
        ms_step, st_stats, graphs = timed_steps([[fused_call(s, rope)] for s in sets], steps,
                                                warmup, torch)
        ms_sep, sep_stats, _ = timed_steps(sep_fns, steps, warmup, torch)
        log(f"{name}{' + rope' if rope else ''}: {ms_step * 1e3:.1f} us per step "
            f"({ms_sep * 1e3:.1f} us as separate calls)")
    else:
        ms_step, st_stats, graphs = timed_steps(sep_fns, steps, warmup, torch)
        log(f"{name}{' + rope' if rope else ''}: {ms_step * 1e3:.1f} us per step")

    kern = {}
    reps = KERNEL_REPS
    for ki, (kname, _) in enumerate(calls[0]):
        fns = [calls[i][ki][1] for i in range(n_sets)]
        kern[kname] = {k: v * 1e3 for k, v in time_kernel(fns, reps, evict, torch).items()}
    # restore a consistent state (the index buffer is rebuilt by a full step)
    graphs[0].replay()
    torch.cuda.synchronize()

    parity = parity_report(sets[0], wl, oracle_outputs) if not rope else None
    idx = sets[0].idx.cpu().numpy()
    pairs = None
    if wl.mode == "prefill":
        cand = sets[0].cand.cpu().numpy()
        pairs = 0
        for t in range(wl.n_tokens):
            n = min(wl.n_rows, (t + 1) // wl.ratio)
            blocks = np.repeat(cand[t].astype(bool), wl.cand_block)[:n]
            pairs += int(blocks.sum())
    work = algorithmic(wl, host_idx=idx, valid_pairs=pairs, rope=rope)
    del sets, calls, sep_fns, graphs
    torch.cuda.empty_cache()
    return {"wl": wl, "ms_step": ms_step, "step_stats": st_stats, "kern": kern, "work": work,
            "ms_sep": ms_sep, "sep_stats": sep_stats, "parity": parity}


def time_steps_only(name, steps, warmup, n_sets, torch, device, rope=False, separate=False):
    """The K graph-replayed steps of run_workload alone (the same staging,
    input sets and step form), nothing else launched in between."""
    wl = WL.WORKLOADS[name]
    if wl.mode == "decode":
        buf0, _ = stage_decode(wl, device)
        buf0.pos = wl.start_pos
        buf0.pos_dev = torch.full((wl.batch,), wl.start_pos, dtype=torch.int32, device=device)
    else:
        buf0, _ = stage_prefill(wl, device)
    if rope:
        attach_rope(buf0, wl, device)
    sets = [buf0] + [clone_buffers(buf0) for _ in range(n_sets - 1)]
    for s in sets:
        s.pos = getattr(buf0, "pos", 0)
    if wl.mode == "decode" and not separate:
        fns, form = [[fused_call(s, rope)] for s in sets], "v41_decode_step"
    else:
        fns = [[f for _, f in step_calls(s, wl.mode, rope)] for s in sets]
        form = "separate calls"
    ms_step, st_stats, _ = timed_steps(fns, steps, warmup, torch)
    log(f"{name}: {ms_step * 1e3:.1f} us per step ({form}, steps only)")
    return {"ms_step": ms_step, "step_stats": st_stats, "form": form}


# Sources of each kernel: a stored traffic figure holds only while they are
# unchanged.
KERNEL_SOURCES = {
    "indexer_scores": ("v41_indexer.hip", "v41_common.h"),
    "sparse_attn_sink": ("v41_attn.hip", "v41_common.h"),
    "topk_select": ("v41_topk.hip", "v41_common.h"),
}


def source_digest(kname):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kname, ()):
        with open(os.path.join(ROOT, "indexer_top_sink_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kname, workload):
    """HBM bytes per launch from profiles/hbm_traffic.json (FETCH_SIZE + WRITE_SIZE
    counter runs scaled by a plain copy of known size), or None when absent or
    taken on other sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    for r in recs:
        if r["kernel"] == kname and r["workload"] == workload and \
                r["source_sha256"] == source_digest(kname):
            return r["bytes_per_launch"]
    return None


def roofline_entry(kname, work, kt, bound, workload=None, ceilings=None):
    """Roofline of one kernel: algorithmic bytes (flops) per launch over its
    mean launch time; kt holds the mean / p50 / p90 launch times in us."""
    w = work[kname]
    us = kt["mean"]
    if bound == "hbm":
        achieved = w["bytes"] / (us * 1e-6) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
        measured = ceilings.get("hbm_GBs") if ceilings else None
    else:
        achieved = w["flops"] / (us * 1e-6) / 1e12
        peak, unit = BF16_PEAK_TFLOPS, "TFLOP/s"
        measured = ceilings.get("mfma_bf16_TFLOPs") if ceilings else None
    traffic = measured_traffic(kname, workload) if workload else None
    return {"kernel": kname, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
            "frac_of_measured": round(achieved / measured, 4) if measured else None,
            "avg_us": round(us, 2), "p50_us": round(kt["p50"], 2), "p90_us": round(kt["p90"], 2),
            "algorithmic_bytes": w["bytes"], "algorithmic_flops": w["flops"]}


def us_stats(st):
    return {k: round(v * 1e3, 2) for k, v in st.items()}


def decode_summary(r, ceilings):
    """A decode workload's line: throughput, step time distribution, and the
    roofline of each timed kernel (the longest as `roofline`)."""
    wl, kern, work = r["wl"], r["kern"], r["work"]
    dominant = max(kern, key=lambda k: kern[k]["mean"])
    return {
        "value": round(wl.queries / (r["ms_step"] * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(r["ms_step"], 5), "step_us": us_stats(r["step_stats"]),
        "roofline": roofline_entry(dominant, work, kern[dominant], "hbm", wl.name, ceilings),
        "kernels": {k: roofline_entry(k, work, kern[k], "hbm", wl.name, ceilings)
                    for k in kern},
        "path_hbm_frac": path_frac(r),
        "ms_per_step_separate_calls": (round(r["ms_sep"], 5) if r["ms_sep"] is not None
                                       else None)}


def path_frac(r):
    """Indexer + attention together: their algorithmic bytes over their summed
    mean launch times, as a fraction of the published HBM peak."""
    k, w = r["kern"], r["work"]
    names = [n for n in ("indexer_scores", "sparse_attn_sink") if n in k]
    nbytes = sum(w[n]["bytes"] for n in names)
    us = sum(k[n]["mean"] for n in names)
    return {"kernels": names, "bytes": nbytes, "us": round(us, 2),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=SECONDARY_WARMUP,
                    help="untimed warm-up steps before the K timed ones (the default carries "
                         "the GPU past its clock ramp)")
    ap.add_argument("--workload", default="decode64", choices=sorted(WL.WORKLOADS))
    ap.add_argument("--input-sets", type=int, default=4)
    ap.add_argument("--rope", action="store_true",
                    help="make the rotary epilogue (q rotation; kv rotation + fp8 + ring "
                         "write) part of the timed step")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time a decode step as the separate calls instead of one "
                         "v41_decode_step call")
    ap.add_argument("--output-side", action="store_true",
                    help="time only the output side (inverse rotation, wo_a, wo_b) at decode64 "
                         "and prefill sizes and print that as the JSON line")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the graph-replayed steps of the workload (no per-kernel "
                         "cache-cold timing, ceilings, CPU leg or secondary lines), for a "
                         "kernel trace of the step as it runs")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="first copy MB megabytes device to device three times (the "
                         "known-size kernel that scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); each GPU would "
              "take its own shard of sequences or tokens with no exchange, so run one "
              "process per GPU", file=sys.stderr)
        sys.exit(2)
    wl = WL.WORKLOADS[args.workload]

    # the oracle first, before anything touches the GPU (its pool forks)
    cpu = None
    oracle_out = {}
    if not args.no_cpu_baseline and not args.output_side and not args.step_only:
        t0 = time.time()
        cpu = cpu_baseline(wl)
        oracle_out[wl.name] = cpu.pop("_outputs")
        log(f"cpu baseline in {time.time() - t0:.1f}s: {cpu['value']:.2f} tokens/s on "
            f"{cpu['cores']} processes, {cpu['single_thread']['value']:.2f} on one thread")
    # the same two legs for the secondary workloads, on a smaller budget
    cpu_sec = {}
    if cpu is not None and not args.no_secondary:
        for name in ("prefill", "decode16"):
            if name == wl.name:
                continue
            t0 = time.time()
            cpu_sec[name] = cpu_baseline(WL.WORKLOADS[name], budget_s=5.0)
            oracle_out[name] = cpu_sec[name].pop("_outputs")
            log(f"cpu baseline {name} in {time.time() - t0:.1f}s: "
                f"{cpu_sec[name]['value']:.2f} tokens/s on {cpu_sec[name]['cores']} processes")

    import torch
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    from indexer_top_sink_amd import v41
    v41.load()
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read and {n} written per copy")
        del src, dst

    if args.output_side:
        res = {"decode64": time_grouped_output(torch, device, args.steps, 64),
               "prefill": time_grouped_output(torch, device, args.steps, 2048)}
        print(json.dumps({"metric": "output side us per step (inverse rotation, wo_a, wo_b)",
                          "value": res["decode64"]["us_per_step"], "unit": "us",
                          "higher_is_better": False, "data": "synthetic", "detail": res}),
              flush=True)
        return
    if args.step_only:
        r = time_steps_only(args.workload, args.steps, args.warmup, args.input_sets, torch,
                            device, rope=args.rope, separate=args.separate_calls)
        print(json.dumps({"metric": "us per step (graph-replayed steps only)",
                          "value": round(r["ms_step"] * 1e3, 2), "unit": "us",
                          "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": wl.name, "steps": args.steps,
                                     "input_sets": args.input_sets,
                                     "step_form": r["form"]},
                          "step_us": us_stats(r["step_stats"])}), flush=True)
        return
    ceilings = measured_ceilings(torch, device)
    log(f"measured ceilings: {ceilings}")
    evict = CacheEvictor(torch, device)
    r = run_workload(args.workload, args.steps, args.warmup, args.input_sets, torch, device,
                     evict, rope=args.rope, separate=args.separate_calls,
                     oracle_outputs=oracle_out.get(wl.name))
    kern, work, ms_step = r["kern"], r["work"], r["ms_step"]
    tokens = wl.queries
    value = tokens / (ms_step * 1e-3)
    # the dominant kernel is the one that takes the most time; decode moves
    # bytes (HBM bound), a prefill chunk multiplies (MFMA bound)
    dominant = max(kern, key=lambda k: kern[k]["mean"])
    bound = "mfma" if wl.mode == "prefill" else "hbm"
    roof = roofline_entry(dominant, work, kern[dominant], bound, wl.name, ceilings)
    others = {k: roofline_entry(k, work, kern[k], bound, wl.name, ceilings)
              for k in kern if k != dominant}

    step_bytes = sum(v["bytes"] for v in work.values())
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": wl.mode, "batch": wl.batch,
                   "tokens_per_step": tokens, "position": wl.start_pos,
                   "compressed_rows": wl.n_rows, "heads": wl.n_heads,
                   "head_dim": wl.head_dim, "window": wl.window,
                   "index_heads": wl.index_heads, "index_dim": wl.index_dim,
                   "topk": wl.topk, "ratio": wl.ratio, "hip_graph": True,
                   "input_sets": args.input_sets, "rope_epilogue": bool(args.rope),
                   "step_form": ("separate calls" if args.separate_calls or wl.mode != "decode"
                                 else "v41_decode_step"),
                   "secondary_warmup_steps": SECONDARY_WARMUP,
                   "kernel_timing": "each kernel launched once per input set, back to back, "
                                    "after a 1 GiB read that evicts the 256 MB last-level "
                                    "cache; events around the launches"},
        "step_us": us_stats(r["step_stats"]),
        "roofline": roof,
        "roofline_other": others,
        "measured_ceilings": ceilings,
        "step_hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "ms_per_step_separate_calls": round(r["ms_sep"], 5) if r["ms_sep"] is not None else None,
        "kernels_us": {k: round(v["mean"], 2) for k, v in kern.items()},
        "parity": r["parity"],
    }
    if wl.mode == "decode":
        out["path_hbm_frac"] = path_frac(r)
    sec = out.setdefault("secondary", {}) if not args.no_secondary else {}
    if not args.no_secondary and wl.name != "prefill":
        p = run_workload("prefill", max(12, args.steps // 2), SECONDARY_WARMUP, args.input_sets,
                         torch, device, evict, oracle_outputs=oracle_out.get("prefill"))
        pw, pk, pwork = p["wl"], p["kern"], p["work"]
        sec["prefill"] = {
            "value": round(pw.n_tokens / (p["ms_step"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(p["ms_step"], 5), "step_us": us_stats(p["step_stats"]),
            "roofline": roofline_entry("sparse_attn_sink", pwork, pk["sparse_attn_sink"],
                                       "mfma", pw.name, ceilings),
            "indexer_roofline": roofline_entry("indexer_scores", pwork, pk["indexer_scores"],
                                               "mfma", pw.name, ceilings),
            "kernels_us": {k: round(v["mean"], 2) for k, v in pk.items()},
            "parity": p["parity"]}
        if "prefill" in cpu_sec:
            sec["prefill"]["cpu_baseline"] = cpu_sec["prefill"]
    if not args.no_secondary and wl.name != "decode16":
        # 16 sequences at context 131072 with the planted ties
        d = run_workload("decode16", args.steps, SECONDARY_WARMUP, args.input_sets, torch,
                         device, evict, separate=args.separate_calls,
                         oracle_outputs=oracle_out.get("decode16"))
        sec["decode16"] = decode_summary(d, ceilings)
        sec["decode16"]["parity"] = d["parity"]
        if "decode16" in cpu_sec:
            sec["decode16"]["cpu_baseline"] = cpu_sec["decode16"]
    if not args.no_secondary and wl.name != "decode1":
        # one sequence at context 4096: the step's latency floor (its 1 MB of
        # data stays in the last-level cache between steps)
        l = run_workload("decode1", args.steps, SECONDARY_WARMUP, args.input_sets, torch, device,
                         evict, separate=args.separate_calls)
        sec["decode1_latency"] = {
            "us_per_step": round(l["ms_step"] * 1e3, 2), "step_us": us_stats(l["step_stats"]),
            "us_per_step_separate_calls": (round(l["ms_sep"] * 1e3, 2)
                                           if l["ms_sep"] is not None else None),
            "kernels_us": {k: round(v["mean"], 2) for k, v in l["kern"].items()}}
    if not args.no_secondary:
        sec["candidate_blocks"] = time_candidate_blocks(torch, device, args.steps)
        sec["grouped_output"] = {
            "decode64": time_grouped_output(torch, device, args.steps, 64),
            "prefill": time_grouped_output(torch, device, args.steps, 2048)}
    if not args.no_secondary and not args.rope:
        # the same step with the rotary epilogue in front (pre-rotation q and kv)
        rr = run_workload(wl.name, args.steps, SECONDARY_WARMUP, args.input_sets, torch, device,
                          evict, rope=True, separate=args.separate_calls)
        rw, rk, rwork = rr["wl"], rr["kern"], rr["work"]
        sec["with_rope_epilogue"] = {
            "value": round(rw.queries / (rr["ms_step"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(rr["ms_step"], 5),
            "ms_per_step_separate_calls": (round(rr["ms_sep"], 5) if rr["ms_sep"] is not None
                                           else None),
            "rope_rows": roofline_entry("rope_rows", rwork, rk["rope_rows"], "hbm", rw.name),
            "rope_fp8_rows": roofline_entry("rope_fp8_rows", rwork, rk["rope_fp8_rows"], "hbm",
                                            rw.name),
            "kernels_us": {k: round(v["mean"], 2) for k, v in rk.items()}}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
