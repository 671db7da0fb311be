"""GPU parity of whole steps at the workloads' full sizes, staged and launched
exactly as bench.py does (same buffers, same calls), checked against the
oracle: every fp8 row, window index and top-k row bit-exact (top-k on the
GPU's own scores), indexer scores and attention outputs on sampled sequences
or tokens that the oracle computes one by one."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from indexer_top_sink_amd import layer as LY
from inputs import workloads as W
from oracle import layer as OL
from parity import assert_attn_close, assert_scores_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def run_decode(wl):
    buf, host = bench.stage_decode(wl, DEV, keep_host=True)
    buf.pos = wl.start_pos
    for _, f in bench.step_calls(buf, "decode"):
        f()
    torch.cuda.synchronize()
    return buf, host


def check_decode(wl, buf, host, sample):
    W_, D = wl.window, wl.head_dim
    sink = W.layer_sink(wl)
    ring = LY.to_numpy_bf16(buf.ring)
    idx = buf.idx.cpu().numpy()
    scores = buf.scores.cpu().numpy()
    out = LY.to_numpy_bf16(buf.out)
    slot = wl.start_pos % W_
    want_widx = O.window_idx(wl.start_pos, 1, W_)[0]
    for b in range(wl.batch):
        d = host[b]
        # ring: earlier rows and the new row, all through the fp8 round trip
        want_ring = O.fp8_round_rows(d["ring_raw"])
        want_ring[slot] = O.fp8_round_rows(d["kv_new"])[0]
        assert np.array_equal(ring[b], want_ring), f"ring of sequence {b}"
        assert np.array_equal(idx[b, :W_], want_widx), f"window of sequence {b}"
    # top-k of every row, on the GPU's scores
    assert np.array_equal(idx[:, W_:], O.topk(scores, wl.topk, W_)), "top-k"
    for b in sample:
        d = host[b]
        say(wl.name, "sequence", b)
        ora_s = O.indexer_scores(d["qI"], d["kI"], d["w"], wl.start_pos, wl.ratio)
        assert_scores_close(scores[b:b + 1], ora_s, f"{wl.name} scores b={b}")
        # informational: rows whose selected sets differ in an all-oracle chain
        ora_sel = O.topk(ora_s, wl.topk, W_)
        diff = len(set(ora_sel[0].tolist()) ^ set(idx[b, W_:].tolist()))
        print(f"[info] {wl.name} b={b}: all-oracle vs GPU selection symmetric difference {diff}",
              flush=True)
        ora_o = O.sparse_attn(d["q"], ring[b], d["latent"], idx[b:b + 1], sink, wl.scale)
        assert_attn_close(out[b:b + 1], ora_o, f"{wl.name} attention b={b}")


def test_decode1_full():
    wl = W.WORKLOADS["decode1"]
    say("decode1 full")
    buf, host = run_decode(wl)
    check_decode(wl, buf, host, sample=[0])


def test_decode64_sampled():
    wl = W.WORKLOADS["decode64"]
    say("decode64 staging")
    buf, host = run_decode(wl)
    check_decode(wl, buf, host, sample=[0, 17, 42, 63])


def test_decode16_ties():
    wl = W.WORKLOADS["decode16"]
    say("decode16 staging")
    buf, host = run_decode(wl)
    check_decode(wl, buf, host, sample=[0, 9, 15])
    idx = buf.idx.cpu().numpy()[:, wl.window:] - wl.window
    scores = buf.scores.cpu().numpy()
    src = W.tie_source_rows()
    for b in range(8):
        # the 301-way tie group straddles the k-th place: some of it selected,
        # some not, and the selected members are its lowest positions
        tie = scores[b] == scores[b, src[b]]
        members = np.nonzero(tie)[0]
        chosen = np.intersect1d(members, idx[b])
        assert 301 <= members.size and 0 < chosen.size < members.size, b
        assert chosen.max() < np.setdiff1d(members, chosen).min(), b
    for b in range(8, 12):
        # ~32k zero scores: the positive ones first, then the lowest zeros
        zeros = np.nonzero(scores[b] == 0)[0]
        assert zeros.size > 30000
        sel_zero = np.intersect1d(zeros, idx[b])
        assert np.array_equal(sel_zero, zeros[:sel_zero.size]), b


def test_prefill_sampled():
    wl = W.WORKLOADS["prefill"]
    say("prefill staging")
    buf, d = bench.stage_prefill(wl, DEV, keep_host=True)
    for _, f in bench.step_calls(buf, "prefill"):
        f()
    torch.cuda.synchronize()
    T, W_, L = wl.n_tokens, wl.window, wl.n_rows
    sink = W.layer_sink(wl)
    rows_a = LY.to_numpy_bf16(buf.rows_a)
    want_rows = O.fp8_round_rows(d["kv_chunk"])
    assert np.array_equal(rows_a, want_rows), "fp8 rows"
    ring = O.WindowCache(W_, wl.head_dim)
    ring.prefill(want_rows)
    assert np.array_equal(LY.to_numpy_bf16(buf.ring), ring.rows), "ring"
    idx = buf.idx.cpu().numpy()
    assert np.array_equal(idx[:, :W_], O.window_idx(0, T, W_)), "window"
    scores = buf.scores.cpu().numpy()
    assert np.array_equal(idx[:, W_:], O.topk(scores, wl.topk, T)), "top-k"
    # -1 padding: every token has fewer than k visible unmasked positions
    assert (idx[:, W_:] == -1).any(axis=1).all()
    toks = [0, 1, 3, 4, 126, 127, 128, 1000, 2046, 2047]
    toks += sorted(np.random.default_rng(5).choice(np.arange(5, 2046), 10, replace=False))
    say("prefill tokens", toks)
    ora_s = O.indexer_scores(d["qI"], d["kI"], d["w"], 0, wl.ratio, cand=d["cand"],
                             cand_block=wl.cand_block, tokens=toks)
    assert_scores_close(scores[toks], ora_s, "prefill scores")
    out = LY.to_numpy_bf16(buf.out)
    ora_o = O.sparse_attn(d["q"][toks], rows_a, d["latent"], idx[toks], sink, wl.scale)
    assert_attn_close(out[toks], ora_o, "prefill attention")


def test_tiny_pair_chain():
    """The tiny pair through the smoke path (ratio-4 layer) and the ratio-0
    layer's prefill and decodes through one ring."""
    import __graft_entry__
    __graft_entry__.smoke()
    wl = W.TINY
    d = W.tiny_inputs(0)
    geo = LY.Geometry(n_heads=wl.n_heads, head_dim=wl.head_dim, window=wl.window,
                      index_heads=wl.index_heads, index_dim=wl.index_dim, topk=wl.topk,
                      ratio=0, scale=wl.scale)
    T, D, W_ = wl.n_tokens, wl.head_dim, wl.window
    pre = LY.alloc_prefill(geo, T, 0, 0, 1, DEV)
    pre.kv_chunk.copy_(LY.to_device_bf16(d["kv_chunk"], DEV))
    pre.q.copy_(LY.to_device_bf16(d["q"], DEV))
    pre.sink.copy_(torch.from_numpy(d["sink"]).to(DEV))
    LY.prefill_chunk(pre)
    torch.cuda.synchronize()
    ring = O.WindowCache(W_, D)
    want = OL.prefill(d["kv_chunk"], d["q"], d["sink"], wl.scale, W_, ring=ring)
    assert np.array_equal(LY.to_numpy_bf16(pre.rows_a), want["rows_a"])
    assert np.array_equal(pre.idx.cpu().numpy(), want["idx"])
    assert_attn_close(LY.to_numpy_bf16(pre.out), want["out"], "tiny ratio-0 prefill")
    dec = LY.alloc_decode(geo, 1, 0, DEV)
    dec.ring[0].copy_(pre.ring)
    dec.sink.copy_(pre.sink)
    for p in W.TINY_DECODE_POSITIONS:
        dec.kv_new[0].copy_(LY.to_device_bf16(d[f"kv_new_{p}"][0], DEV))
        dec.q[0].copy_(LY.to_device_bf16(d[f"q_{p}"][0], DEV))
        LY.decode_step(dec, p)
        torch.cuda.synchronize()
        want = OL.decode(ring, d[f"kv_new_{p}"], p, d[f"q_{p}"], d["sink"], wl.scale)
        assert np.array_equal(LY.to_numpy_bf16(dec.ring[0]), ring.rows)
        assert np.array_equal(dec.idx.cpu().numpy(), want["idx"])
        assert_attn_close(LY.to_numpy_bf16(dec.out), want["out"], f"tiny ratio-0 decode {p}")


# ------------------------------------------------------------------ with the rotary epilogue
def oracle_table_at(buf, wl, positions):
    """The oracle's RoPE table, after checking that the GPU's table rows at
    `positions` are bit-identical to it (then every rotation and fp8 decision
    below is taken on the same numbers on both sides)."""
    gpu = buf.rope.table.cpu().numpy()
    ora = O.rope_table(wl.rope_theta, wl.rope_dim, gpu.shape[0])
    for p in positions:
        assert np.array_equal(gpu[p], ora[p]), f"table row {p} differs from the oracle's"
    return ora


def test_decode64_rope_sampled():
    wl = W.WORKLOADS["decode64"]
    say("decode64 + rope staging")
    buf, host = bench.stage_decode(wl, DEV, keep_host=True)
    buf.pos = wl.start_pos
    bench.attach_rope(buf, wl, DEV)
    for _, f in bench.step_calls(buf, "decode", rope=True):
        f()
    torch.cuda.synchronize()
    p, W_, H, rd = wl.start_pos, wl.window, wl.n_heads, wl.rope_dim
    tab = oracle_table_at(buf, wl, [p])
    sink = W.layer_sink(wl)
    q = LY.to_numpy_bf16(buf.q)
    ring = LY.to_numpy_bf16(buf.ring)
    idx = buf.idx.cpu().numpy()
    out = LY.to_numpy_bf16(buf.out)
    slot = p % W_
    q_host = np.stack([host[b]["q"][0] for b in range(wl.batch)])
    want_q = O.rope_rows(q_host, tab, np.full(wl.batch * H, p), rd).reshape(q_host.shape)
    assert np.array_equal(q, want_q), "rotated q"
    for b in range(wl.batch):
        want_ring = O.fp8_round_rows(host[b]["ring_raw"])
        want_ring[slot] = O.rope_fp8_rows(host[b]["kv_new"], tab, [p], rd)[0]
        assert np.array_equal(ring[b], want_ring), f"ring of sequence {b}"
    assert np.array_equal(idx[:, W_:], O.topk(buf.scores.cpu().numpy(), wl.topk, W_)), "top-k"
    for b in (0, 31, 63):
        say("decode64 + rope attention", b)
        ora_o = O.sparse_attn(want_q[b:b + 1], ring[b], host[b]["latent"], idx[b:b + 1], sink,
                              wl.scale)
        assert_attn_close(out[b:b + 1], ora_o, f"decode64 + rope attention b={b}")


def test_prefill_rope_sampled():
    wl = W.WORKLOADS["prefill"]
    say("prefill + rope staging")
    buf, d = bench.stage_prefill(wl, DEV, keep_host=True)
    bench.attach_rope(buf, wl, DEV)
    for _, f in bench.step_calls(buf, "prefill", rope=True):
        f()
    torch.cuda.synchronize()
    T, W_, H, rd = wl.n_tokens, wl.window, wl.n_heads, wl.rope_dim
    tab = oracle_table_at(buf, wl, range(T))
    want_q = O.rope_rows(d["q"], tab, np.repeat(np.arange(T), H), rd).reshape(d["q"].shape)
    assert np.array_equal(LY.to_numpy_bf16(buf.q), want_q), "rotated q"
    want_rows = O.rope_fp8_rows(d["kv_chunk"], tab, np.arange(T), rd)
    rows_a = LY.to_numpy_bf16(buf.rows_a)
    assert np.array_equal(rows_a, want_rows), "rotated fp8 rows"
    ring = O.WindowCache(W_, wl.head_dim)
    ring.prefill(want_rows)
    assert np.array_equal(LY.to_numpy_bf16(buf.ring), ring.rows), "ring"
    idx = buf.idx.cpu().numpy()
    toks = [0, 1, 127, 128, 1500, 2047]
    say("prefill + rope tokens", toks)
    out = LY.to_numpy_bf16(buf.out)
    ora_o = O.sparse_attn(want_q[toks], rows_a, d["latent"], idx[toks], W.layer_sink(wl),
                          wl.scale)
    assert_attn_close(out[toks], ora_o, "prefill + rope attention")


def test_tiny_ratio0_chain_with_rope():
    """The ratio-0 layer of the tiny pair with the rotary epilogue (RoPE on
    the last 16 values): prefill of 12 tokens, then decodes 12 and 13 through
    one ring, device positions at decode."""
    wl = W.TINY
    d = W.tiny_inputs(0)
    geo = LY.Geometry(n_heads=wl.n_heads, head_dim=wl.head_dim, window=wl.window,
                      index_heads=wl.index_heads, index_dim=wl.index_dim, topk=wl.topk,
                      ratio=0, scale=wl.scale)
    T, D, W_ = wl.n_tokens, wl.head_dim, wl.window
    say("tiny ratio-0 + rope")
    rt = LY.rope_table(wl.rope_theta, wl.rope_dim, 14, DEV)
    tab = O.rope_table(wl.rope_theta, wl.rope_dim, 14)
    assert np.array_equal(rt.table.cpu().numpy(), tab)
    pre = LY.alloc_prefill(geo, T, 0, 0, 1, DEV)
    pre.kv_chunk.copy_(LY.to_device_bf16(d["kv_chunk"], DEV))
    pre.q.copy_(LY.to_device_bf16(d["q"], DEV))
    pre.sink.copy_(torch.from_numpy(d["sink"]).to(DEV))
    LY.prefill_chunk(pre, rope=rt)
    torch.cuda.synchronize()
    ring = O.WindowCache(W_, D)
    want = OL.prefill(d["kv_chunk"], d["q"], d["sink"], wl.scale, W_, ring=ring,
                      rope=(tab, wl.rope_dim))
    assert np.array_equal(LY.to_numpy_bf16(pre.q), want["q"])
    assert np.array_equal(LY.to_numpy_bf16(pre.rows_a), want["rows_a"])
    assert np.array_equal(LY.to_numpy_bf16(pre.ring), ring.rows)
    assert_attn_close(LY.to_numpy_bf16(pre.out), want["out"], "tiny ratio-0 + rope prefill")
    dec = LY.alloc_decode(geo, 1, 0, DEV)
    dec.ring[0].copy_(pre.ring)
    dec.sink.copy_(pre.sink)
    pos_dev = torch.zeros(1, dtype=torch.int32, device=DEV)
    for p in W.TINY_DECODE_POSITIONS:
        dec.kv_new[0].copy_(LY.to_device_bf16(d[f"kv_new_{p}"][0], DEV))
        dec.q[0].copy_(LY.to_device_bf16(d[f"q_{p}"][0], DEV))
        pos_dev.fill_(p)
        LY.decode_step(dec, p, rope=rt, pos_dev=pos_dev)
        torch.cuda.synchronize()
        want = OL.decode(ring, d[f"kv_new_{p}"], p, d[f"q_{p}"], d["sink"], wl.scale,
                         rope=(tab, wl.rope_dim))
        assert np.array_equal(LY.to_numpy_bf16(dec.q), want["q"])
        assert np.array_equal(LY.to_numpy_bf16(dec.ring[0]), ring.rows)
        assert_attn_close(LY.to_numpy_bf16(dec.out), want["out"], f"tiny + rope decode {p}")
