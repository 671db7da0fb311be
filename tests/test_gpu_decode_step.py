"""GPU parity of the one-call decode step (v41_decode_step): the same results
as the separate calls, graph replays over consecutive positions read on the
device, sequences at different positions, and the degenerate cases (window
only, no compressed row yet).  Checked against the oracle chain (oracle.layer)
and, where the kernels are deterministic (ring, window and top-k indices,
scores), bit for bit against the separate calls."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from indexer_top_sink_amd import layer as LY
from inputs import synth as S
from inputs import workloads as W
from oracle import layer as OL
from parity import assert_attn_close, assert_scores_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def snapshot(buf):
    return {"ring": LY.to_numpy_bf16(buf.ring), "idx": buf.idx.cpu().numpy(),
            "scores": buf.scores.cpu().numpy(), "out": LY.to_numpy_bf16(buf.out),
            "q": LY.to_numpy_bf16(buf.q)}


@pytest.mark.parametrize("name,rope", [("decode1", False), ("decode64", False),
                                       ("decode64", True), ("decode16", False)])
def test_fused_step_matches_separate_calls(name, rope):
    wl = W.WORKLOADS[name]
    say("fused vs separate", name, "rope" if rope else "")
    buf, host = bench.stage_decode(wl, DEV, keep_host=True)
    buf.pos = wl.start_pos
    if rope:
        bench.attach_rope(buf, wl, DEV)
    twin = bench.clone_buffers(buf)
    for _, f in bench.step_calls(buf, "decode", rope):
        f()
    torch.cuda.synchronize()
    pos_dev = torch.full((wl.batch,), wl.start_pos, dtype=torch.int32, device=DEV)
    LY.decode_step_fused(twin, pos_dev, buf.rope if rope else None)
    torch.cuda.synchronize()
    a, b = snapshot(buf), snapshot(twin)
    for k in ("ring", "idx", "scores", "q"):
        assert np.array_equal(a[k], b[k]), k
    # attention accumulates in a run-dependent order: compare with the oracle
    sink = W.layer_sink(wl)
    for s in sorted({0, wl.batch // 2, wl.batch - 1}):
        ora = O.sparse_attn(b["q"][s:s + 1], b["ring"][s], host[s]["latent"],
                            b["idx"][s:s + 1], sink, wl.scale)
        assert_attn_close(b["out"][s:s + 1], ora, f"{name} fused attention b={s}")


def test_fused_graph_replays_over_positions():
    """One graph [decode step; pos += 1] replayed four times: two sequences
    at different positions (one ring not yet full, one wrapped whose causal
    bound grows from 1023 to 1024 visible rows of 1030 present), with the
    rotary epilogue.  Each replay is checked against the oracle chain."""
    B, H, D, Wn, HI, DI, k, ratio, L, rd = 2, 64, 512, 128, 64, 128, 512, 4, 1030, 64
    p0 = [5, 4093]
    steps = 4
    geo = LY.Geometry(n_heads=H, head_dim=D, window=Wn, index_heads=HI, index_dim=DI, topk=k,
                      ratio=ratio, scale=float(np.float32(1.0 / np.sqrt(D))))
    buf = LY.alloc_decode(geo, B, L, DEV)
    seed = 0x5EED7000
    sink = S.normal_f32(seed, S.TAG_SINK, (H,))
    buf.sink.copy_(torch.from_numpy(sink).to(DEV))
    rings, latent, kI = [], [], []
    for b in range(B):
        r = O.WindowCache(Wn, D)
        raw = O.fp8_round_rows(S.normal_bf16(seed + b, S.TAG_KV_RING, (Wn, D)))
        n_old = min(p0[b], Wn)           # tokens 0 .. p0-1 hold slots before the first step
        for t in range(p0[b] - n_old, p0[b]):
            r.put(raw[t % Wn], t)
        rings.append(r)
        latent.append(S.normal_bf16(seed + b, S.TAG_LATENT, (L, D)))
        kI.append(S.normal_bf16(seed + b, S.TAG_KI, (L, DI)))
        buf.ring[b].copy_(LY.to_device_bf16(r.rows, DEV))
        buf.latent[b].copy_(LY.to_device_bf16(latent[b], DEV))
        buf.kI[b].copy_(LY.to_device_bf16(kI[b], DEV))
    n_tab = max(p0) + steps
    rt = LY.rope_table(10000.0, rd, n_tab, DEV)
    tab = O.rope_table(10000.0, rd, n_tab)
    gtab = rt.table.cpu().numpy()
    for b in range(B):
        for p in range(p0[b], p0[b] + steps):
            assert np.array_equal(gtab[p], tab[p]), p
    pos_dev = torch.tensor(p0, dtype=torch.int32, device=DEV)

    def inputs(step):
        d = []
        for b in range(B):
            s = seed + 100 * (step + 1) + b
            d.append({"q": S.normal_bf16(s, S.TAG_Q, (1, H, D)),
                      "kv_new": S.normal_bf16(s, S.TAG_KV_NEW, (1, D)),
                      "qI": S.normal_bf16(s, S.TAG_QI, (1, HI, DI)),
                      "w": S.uniform_f32(s, S.TAG_W, (1, HI), scale=1.0 / 64)})
        return d

    def load(d):
        for b in range(B):
            buf.q[b].copy_(LY.to_device_bf16(d[b]["q"][0], DEV))
            buf.kv_new[b].copy_(LY.to_device_bf16(d[b]["kv_new"][0], DEV))
            buf.qI[b].copy_(LY.to_device_bf16(d[b]["qI"][0], DEV))
            buf.w[b].copy_(torch.from_numpy(d[b]["w"][0]).to(DEV))

    args = LY.decode_step_args(buf, pos_dev, rt)
    from indexer_top_sink_amd import v41
    # a call with no sequence: the library's one-time device check runs
    # before the capture, and nothing is launched
    v41.v41_decode_step(v41.DecodeStepArgs.make(batch=0, n_heads=1, head_dim=64, window=1,
                                                ratio=0))
    d0 = inputs(0)
    load(d0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        v41.v41_decode_step(args)
        pos_dev.add_(1)
    torch.cuda.synchronize()
    # capture does not run the work: the state is as staged
    assert pos_dev.cpu().tolist() == p0
    for step in range(steps):
        d = d0 if step == 0 else inputs(step)
        if step:
            load(d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(buf)
        assert pos_dev.cpu().tolist() == [p + step + 1 for p in p0]
        for b in range(B):
            p = p0[b] + step
            say("graph replay", step, "sequence", b, "position", p)
            want = OL.decode(rings[b], d[b]["kv_new"], p, d[b]["q"], sink, geo.scale,
                             ratio=ratio, latent=latent[b], kI=kI[b], qI=d[b]["qI"],
                             w=d[b]["w"], k=k, rope=(tab, rd))
            assert np.array_equal(got["ring"][b], rings[b].rows), "ring"
            assert np.array_equal(got["q"][b], want["q"][0]), "rotated q"
            assert np.array_equal(got["idx"][b, :Wn], want["widx"][0]), "window"
            assert_scores_close(got["scores"][b:b + 1], want["scores"], f"scores p={p}")
            gs = got["scores"][b:b + 1]
            assert np.array_equal(got["idx"][b:b + 1, Wn:], O.topk(gs, k, Wn)), "top-k"
            n_vis = min(L, (p + 1) // ratio)
            assert int((got["idx"][b, Wn:] >= 0).sum()) == min(k, n_vis)
            ora = O.sparse_attn(want["q"], rings[b].rows, latent[b], got["idx"][b:b + 1], sink,
                                geo.scale)
            assert_attn_close(got["out"][b:b + 1], ora, f"replay {step} b={b}")


def test_fused_window_only_and_no_compressed_rows():
    """ratio 0 (window only) through the tiny ratio-0 layer's decodes, and a
    ratio-4 step before any compressed row exists (the top-k columns all -1)."""
    wl = W.TINY
    d = W.tiny_inputs(0)
    T, D, Wn = wl.n_tokens, wl.head_dim, wl.window
    geo0 = LY.Geometry(n_heads=wl.n_heads, head_dim=D, window=Wn, index_heads=wl.index_heads,
                       index_dim=wl.index_dim, topk=wl.topk, ratio=0, scale=wl.scale)
    say("fused tiny ratio 0")
    ring = O.WindowCache(Wn, D)
    OL.prefill(d["kv_chunk"], d["q"], d["sink"], wl.scale, Wn, ring=ring)
    dec = LY.alloc_decode(geo0, 1, 0, DEV)
    dec.ring[0].copy_(LY.to_device_bf16(ring.rows, DEV))
    dec.sink.copy_(torch.from_numpy(d["sink"]).to(DEV))
    pos_dev = torch.zeros(1, dtype=torch.int32, device=DEV)
    for p in W.TINY_DECODE_POSITIONS:
        dec.kv_new[0].copy_(LY.to_device_bf16(d[f"kv_new_{p}"][0], DEV))
        dec.q[0].copy_(LY.to_device_bf16(d[f"q_{p}"][0], DEV))
        pos_dev.fill_(p)
        LY.decode_step_fused(dec, pos_dev)
        torch.cuda.synchronize()
        want = OL.decode(ring, d[f"kv_new_{p}"], p, d[f"q_{p}"], d["sink"], wl.scale)
        assert np.array_equal(LY.to_numpy_bf16(dec.ring[0]), ring.rows)
        assert np.array_equal(dec.idx.cpu().numpy(), want["idx"])
        assert_attn_close(LY.to_numpy_bf16(dec.out), want["out"], f"fused tiny decode {p}")

    say("fused ratio 4 with no compressed rows")
    geo4 = LY.Geometry(n_heads=wl.n_heads, head_dim=D, window=Wn, index_heads=wl.index_heads,
                       index_dim=wl.index_dim, topk=wl.topk, ratio=4, scale=wl.scale)
    dec4 = LY.alloc_decode(geo4, 1, 0, DEV)
    dec4.ring[0].copy_(LY.to_device_bf16(ring.rows, DEV))
    dec4.sink.copy_(dec.sink)
    p = 14
    kv = S.normal_bf16(77, S.TAG_KV_NEW, (1, D))
    q = S.normal_bf16(77, S.TAG_Q, (1, wl.n_heads, D))
    dec4.kv_new[0].copy_(LY.to_device_bf16(kv[0], DEV))
    dec4.q[0].copy_(LY.to_device_bf16(q[0], DEV))
    pos_dev.fill_(p)
    LY.decode_step_fused(dec4, pos_dev)
    torch.cuda.synchronize()
    want = OL.decode(ring, kv, p, q, d["sink"], wl.scale)
    idx = dec4.idx.cpu().numpy()
    assert np.array_equal(idx[0, :Wn], want["idx"][0])
    assert np.all(idx[0, Wn:] == -1)
    assert np.array_equal(LY.to_numpy_bf16(dec4.ring[0]), ring.rows)
    assert_attn_close(LY.to_numpy_bf16(dec4.out), want["out"], "fused, no compressed rows")


def test_fused_negative_position_writes_nothing():
    """A sequence with a negative device position writes no ring row, gets an
    empty window and an empty selection, and so an all-zero output; the
    other sequence of the call is unaffected."""
    wl = W.WORKLOADS["decode1"]
    say("fused negative position")
    geo = bench.geometry(wl)
    B, D, Wn, L = 2, wl.head_dim, wl.window, 64
    buf = LY.alloc_decode(geo, B, L, DEV)
    ring0 = O.fp8_round_rows(S.normal_bf16(91, S.TAG_KV_RING, (B, Wn, D)))
    buf.ring.copy_(LY.to_device_bf16(ring0, DEV))
    buf.kv_new.copy_(LY.to_device_bf16(S.normal_bf16(91, S.TAG_KV_NEW, (B, D)), DEV))
    buf.q.copy_(LY.to_device_bf16(S.normal_bf16(91, S.TAG_Q, (B, geo.n_heads, D)), DEV))
    buf.latent.copy_(LY.to_device_bf16(S.normal_bf16(91, S.TAG_LATENT, (B, L, D)), DEV))
    buf.kI.copy_(LY.to_device_bf16(S.normal_bf16(91, S.TAG_KI, (B, L, geo.index_dim)), DEV))
    buf.qI.copy_(LY.to_device_bf16(S.normal_bf16(91, S.TAG_QI, (B, geo.index_heads,
                                                                  geo.index_dim)), DEV))
    buf.w.copy_(torch.from_numpy(S.uniform_f32(91, S.TAG_W, (B, geo.index_heads),
                                               scale=1.0 / 64)).to(DEV))
    buf.sink.copy_(torch.from_numpy(S.normal_f32(91, S.TAG_SINK, (geo.n_heads,))).to(DEV))
    pos_dev = torch.tensor([-3, 200], dtype=torch.int32, device=DEV)
    LY.decode_step_fused(buf, pos_dev)
    torch.cuda.synchronize()
    ring = LY.to_numpy_bf16(buf.ring)
    assert np.array_equal(ring[0], ring0[0])
    assert np.all(buf.idx.cpu().numpy()[0] == -1)
    assert np.all(LY.to_numpy_bf16(buf.out)[0] == 0)
    want_row = O.fp8_round_rows(LY.to_numpy_bf16(buf.kv_new)[1:2])[0]
    assert np.array_equal(ring[1, 200 % Wn], want_row)


def test_fused_long_rows_with_ties():
    """Score rows of 20000 positions (the sampled-threshold select) through the
    decode step: three sequences (one sees 301 positions, fewer than k; one a
    ragged 12345; one all 20000), a 600-way tie group straddling place k in
    the last two (the key at rank 400 copied over 600 visible positions), the
    step run eagerly and as two graph replays.  Every run's selection equals
    the oracle's top-k of the GPU's scores (the same rows each time) and the
    outputs match the oracle attention."""
    from indexer_top_sink_amd import v41
    B, H, D, Wn, HI, DI, k, ratio, L = 3, 16, 128, 128, 64, 128, 512, 4, 20000
    pos = [4 * 301 - 1, 4 * 12345 - 1, 4 * L - 1]
    geo = LY.Geometry(n_heads=H, head_dim=D, window=Wn, index_heads=HI, index_dim=DI, topk=k,
                      ratio=ratio, scale=float(np.float32(1.0 / np.sqrt(D))))
    seed = 0x5EED7100
    rng = np.random.default_rng(7)
    sink = S.normal_f32(seed, S.TAG_SINK, (H,))
    host = []
    for b in range(B):
        s = seed + b
        kI = S.normal_bf16(s, S.TAG_KI, (L, DI))
        qI = S.normal_bf16(s, S.TAG_QI, (HI, DI))
        w = S.uniform_f32(s, S.TAG_W, (HI,), scale=1.0 / 64)
        n_vis = min(L, (pos[b] + 1) // ratio)
        if n_vis > k:
            sc = O.indexer_scores(qI[None], kI, w[None], pos[b], ratio)[0][:n_vis]
            src = int(np.lexsort((np.arange(n_vis), -sc))[400])
            kI[rng.choice(n_vis, 600, replace=False)] = kI[src]
        host.append({"ring": O.fp8_round_rows(S.normal_bf16(s, S.TAG_KV_RING, (Wn, D))),
                     "latent": S.normal_bf16(s, S.TAG_LATENT, (L, D)), "kI": kI,
                     "q": S.normal_bf16(s, S.TAG_Q, (H, D)),
                     "kv_new": S.normal_bf16(s, S.TAG_KV_NEW, (D,)), "qI": qI, "w": w})

    def staged():
        buf = LY.alloc_decode(geo, B, L, DEV)
        buf.sink.copy_(torch.from_numpy(sink).to(DEV))
        for b, h in enumerate(host):
            buf.ring[b].copy_(LY.to_device_bf16(h["ring"], DEV))
            buf.latent[b].copy_(LY.to_device_bf16(h["latent"], DEV))
            buf.kI[b].copy_(LY.to_device_bf16(h["kI"], DEV))
            buf.q[b].copy_(LY.to_device_bf16(h["q"], DEV))
            buf.kv_new[b].copy_(LY.to_device_bf16(h["kv_new"], DEV))
            buf.qI[b].copy_(LY.to_device_bf16(h["qI"], DEV))
            buf.w[b].copy_(torch.from_numpy(h["w"]).to(DEV))
        return buf

    pos_dev = torch.tensor(pos, dtype=torch.int32, device=DEV)
    buf = staged()
    args = LY.decode_step_args(buf, pos_dev, None)
    v41.v41_decode_step(args)                       # eager, then two replays
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        v41.v41_decode_step(args)
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        if rep:
            buf.idx.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
        got = snapshot(buf)
        say("long rows with ties, run", rep)
        assert np.array_equal(got["idx"][:, Wn:], O.topk(got["scores"], k, Wn)), rep
        for b in range(B):
            n_vis = min(L, (pos[b] + 1) // ratio)
            assert int((got["idx"][b, Wn:] >= 0).sum()) == min(k, n_vis)
        results.append(got["idx"])
    assert all(np.array_equal(results[0], r) for r in results[1:])
    # the tie groups straddle place k, and their chosen members are the lowest
    for b in (1, 2):
        sc = got["scores"][b]
        vals, counts = np.unique(sc[np.isfinite(sc)], return_counts=True)
        members = np.nonzero(sc == vals[np.argmax(counts)])[0]
        chosen = np.intersect1d(members, got["idx"][b, Wn:] - Wn)
        assert members.size >= 600 and 0 < chosen.size < members.size, b
        assert chosen.max() < np.setdiff1d(members, chosen).min(), b
    for b in range(B):
        ora = O.sparse_attn(got["q"][b:b + 1], got["ring"][b], host[b]["latent"],
                            got["idx"][b:b + 1], sink, geo.scale)
        assert_attn_close(got["out"][b:b + 1], ora, f"long-row step attention b={b}")
