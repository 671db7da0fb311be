"""GPU parity of each libv41 call against the oracle, at sizes the oracle
finishes in seconds that span several tiles and a ragged tail, plus edge
cases (empty, ragged, degenerate).  Calls go through the C ABI binding."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from inputs import synth as S
from parity import assert_attn_close, assert_scores_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def v41():
    from indexer_top_sink_amd import v41 as m
    m.load()
    return m


def say(*a):
    print("[case]", *a, flush=True)


def up16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
    return t.to(DEV)


def down16(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def bf16_of(x):
    return S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ fp8
def all_finite_bf16_blocks():
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = S.bf16_bits_to_f32(allb)
    fin = allb[np.isfinite(x)]
    n = (fin.size // 32) * 32
    srt = fin[np.argsort(x[np.isfinite(x)], kind="stable")][:n]
    rng = np.random.default_rng(11)
    return np.concatenate([srt, rng.permutation(fin)[:n]]).reshape(-1, 512)


def test_fp8_exhaustive_bf16(v41):
    rows = all_finite_bf16_blocks()
    say("fp8 exhaustive", rows.shape)
    d_in = up16(rows)
    d_out = torch.empty_like(d_in)
    v41.v41_fp8_round_rows(d_in, 512, d_out, 512, rows.shape[0], 512)
    assert np.array_equal(down16(d_out), O.fp8_round_rows(rows))


@pytest.mark.parametrize("rows,row_len,in_ld,out_ld", [(1, 32, 32, 32), (7, 64, 72, 80),
                                                       (2048, 512, 512, 512), (3, 96, 96, 104)])
def test_fp8_strided(v41, rows, row_len, in_ld, out_ld):
    say("fp8 strided", rows, row_len, in_ld, out_ld)
    rng = np.random.default_rng(rows)
    x = bf16_of(rng.standard_normal((rows, in_ld)) * np.exp(rng.uniform(-20, 20, (rows, 1))))
    d_in = up16(x)
    d_out = torch.full((rows, out_ld), 0x1234, dtype=torch.int16, device=DEV)
    v41.v41_fp8_round_rows(d_in, in_ld, d_out, out_ld, rows, row_len)
    got = down16(d_out)
    assert np.array_equal(got[:, :row_len], O.fp8_round_rows(x[:, :row_len]))
    assert np.all(got[:, row_len:] == 0x1234)


def test_fp8_in_place_and_ring(v41):
    T, D, W = 12, 64, 8
    say("fp8 ring", T, D, W)
    rng = np.random.default_rng(5)
    x = bf16_of(rng.standard_normal((T, D)))
    d = up16(x)
    ring = torch.zeros(W, D, dtype=torch.int16, device=DEV)
    v41.v41_fp8_round_rows(d, D, d, D, T, D, ring, W, 0)
    want = O.fp8_round_rows(x)
    assert np.array_equal(down16(d), want)
    cache = O.WindowCache(W, D)
    cache.prefill(want)
    assert np.array_equal(down16(ring), cache.rows)
    assert cache.token.tolist() == [8, 9, 10, 11, 4, 5, 6, 7]


def test_fp8_zero_rows(v41):
    d = torch.zeros(1, 32, dtype=torch.int16, device=DEV)
    v41.v41_fp8_round_rows(d, 32, d, 32, 0, 32)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ window
@pytest.mark.parametrize("start,T,W,B", [(0, 1, 8, 1), (0, 12, 8, 1), (0, 300, 128, 2),
                                         (0, 2048, 128, 1), (12, 1, 8, 3), (13, 1, 8, 1),
                                         (3, 1, 8, 2), (127, 1, 128, 1), (32767, 1, 128, 64),
                                         (131071, 1, 128, 16)])
def test_window(v41, start, T, W, B):
    say("window", start, T, W, B)
    cols = min(T, W) if start == 0 else W
    ld = cols + 5
    idx = torch.full((B, T, ld), -7, dtype=torch.int32, device=DEV)
    got_cols = v41.v41_window_idx(start, T, W, B, idx, ld, T * ld)
    torch.cuda.synchronize()
    assert got_cols == cols
    g = idx.cpu().numpy()
    want = O.window_idx(start, T, W)
    for b in range(B):
        assert np.array_equal(g[b, :, :cols], want)
    assert np.all(g[:, :, cols:] == -7)


# ------------------------------------------------------------------ indexer
def run_indexer(v41, qI, kI, w, start, ratio, cand=None, cand_block=1, B=1, T=None):
    """qI [B*T, HI, DI], kI [B, L, DI], w [B*T, HI]"""
    Q, HI, DI = qI.shape
    L = kI.shape[1]
    T = Q // B if T is None else T
    d_s = torch.full((Q, L + 3), 7.0, dtype=torch.float32, device=DEV)
    dc = torch.from_numpy(cand).to(DEV) if cand is not None else None
    v41.v41_indexer_scores(up16(qI), up16(kI), L * DI, torch.from_numpy(w).to(DEV), dc,
                           cand.shape[1] if cand is not None else 0, cand_block, B, T, start,
                           ratio, HI, DI, L, d_s, L + 3)
    torch.cuda.synchronize()
    got = d_s.cpu().numpy()
    assert np.all(got[:, L:] == 7.0)
    return got[:, :L]


@pytest.mark.parametrize("HI,DI,L,start,ratio,T,B", [
    (64, 128, 1000, 4095, 4, 1, 1),     # decode, ragged tail
    (64, 128, 333, 10 ** 6, 1, 1, 3),   # batch of decodes
    (64, 128, 1000, 4095, 4, 1, 8),     # eight decodes: each query's workgroups on one XCD
    (2, 32, 4, 0, 4, 12, 1),            # the tiny layer's prefill
    (17, 64, 97, 0, 4, 400, 1),         # odd head count, causal prefill
    (1, 32, 50, 10 ** 6, 1, 1, 1),
    (48, 128, 512, 0, 4, 64, 1),
    (64, 128, 300, 0, 4, 13, 2),        # two sequences of 13 tokens
    (16, 64, 200, 0, 2, 7, 3),          # three sequences of seven tokens
    (64, 128, 40, 0, 1, 2, 1),          # two tokens
    (64, 128, 20, 0, 1, 50, 1),         # the causal bound capped at the row count
    # a thousand queries and more over short rows (one workgroup per query)
    (17, 64, 97, 0, 4, 1030, 1),        # odd heads
    (64, 128, 256, 0, 4, 1024, 1),
    (4, 32, 1000, 0, 1, 1100, 1),       # 4 heads: near-cancelling scores
    (16, 64, 200, 0, 2, 600, 2),        # two sequences of 600 tokens
])
def test_indexer_parity(v41, HI, DI, L, start, ratio, T, B):
    say("indexer", HI, DI, L, start, ratio, T, B)
    rng = np.random.default_rng(HI * 1000 + L)
    qI = bf16_of(rng.standard_normal((B * T, HI, DI)))
    kI = bf16_of(rng.standard_normal((B, L, DI)))
    w = (rng.uniform(0, 1, (B * T, HI)) / 8).astype(np.float32)
    got = run_indexer(v41, qI, kI, w, start, ratio, B=B, T=T)
    for b in range(B):
        qb, wb = qI[b * T:(b + 1) * T], w[b * T:(b + 1) * T]
        ora = O.indexer_scores(qb, kI[b], wb, start, ratio)
        assert_scores_close(got[b * T:(b + 1) * T], ora, f"indexer b={b}",
                            operands=(qb, kI[b], wb, range(T)))


def test_indexer_candidate_mask(v41):
    T, HI, DI, L, blk = 256, 64, 128, 64, 8
    say("indexer mask", T, L, blk)
    rng = np.random.default_rng(77)
    qI = bf16_of(rng.standard_normal((T, HI, DI)))
    kI = bf16_of(rng.standard_normal((1, L, DI)))
    w = (rng.uniform(0, 1, (T, HI)) / 64).astype(np.float32)
    cand = (rng.uniform(size=(T, L // blk)) < 0.5).astype(np.uint8)
    got = run_indexer(v41, qI, kI, w, 0, 4, cand=cand, cand_block=blk)
    ora = O.indexer_scores(qI, kI[0], w, 0, 4, cand=cand, cand_block=blk)
    assert_scores_close(got, ora, "masked", operands=(qI, kI[0], w, range(T)))


@pytest.mark.parametrize("blk", [1, 5, 8, 16, 24, 64])
def test_indexer_mask_blocks(v41, blk):
    """Mask blocks shorter than, equal to, longer than and not aligned with
    the kernel's 16-key blocks: a key block is skipped only when none of its
    visible positions is unmasked, and a partly masked one scores -inf at
    its masked positions."""
    T, HI, DI, L = 300, 64, 128, 1000
    say("indexer mask blocks", blk)
    rng = np.random.default_rng(100 + blk)
    qI = bf16_of(rng.standard_normal((T, HI, DI)))
    kI = bf16_of(rng.standard_normal((1, L, DI)))
    w = (rng.uniform(0, 1, (T, HI)) / 64).astype(np.float32)
    nb = (L + blk - 1) // blk
    cand = (rng.uniform(size=(T, nb)) < 0.4).astype(np.uint8)
    got = run_indexer(v41, qI, kI, w, 0, 1, cand=cand, cand_block=blk)
    ora = O.indexer_scores(qI, kI[0], w, 0, 1, cand=cand, cand_block=blk)
    assert_scores_close(got, ora, f"mask blocks of {blk}", operands=(qI, kI[0], w, range(T)))


@pytest.mark.parametrize("blk", [5, 16, 64])
def test_indexer_mask_many_queries(v41, blk):
    """The masked stream for 1100 tokens over 1000 keys at ratio 1 (every
    query in a workgroup of its own, up to 63 key blocks each): masked and
    invisible blocks written -inf, a token's blocks split over its four
    wavefronts' live lists."""
    T, HI, DI, L = 1100, 64, 128, 1000
    say("indexer mask, many queries", blk)
    rng = np.random.default_rng(300 + blk)
    qI = bf16_of(rng.standard_normal((T, HI, DI)))
    kI = bf16_of(rng.standard_normal((1, L, DI)))
    w = (rng.uniform(0, 1, (T, HI)) / 64).astype(np.float32)
    nb = (L + blk - 1) // blk
    cand = (rng.uniform(size=(T, nb)) < 0.4).astype(np.uint8)
    toks = list(range(0, 40)) + [255, 256, 511, 777, 998, 999, 1000, 1098, 1099]
    got = run_indexer(v41, qI, kI, w, 0, 1, cand=cand, cand_block=blk)[toks]
    ora = O.indexer_scores(qI, kI[0], w, 0, 1, cand=cand, cand_block=blk, tokens=toks)
    assert_scores_close(got, ora, f"masked, many queries, blocks of {blk}",
                        operands=(qI, kI[0], w, toks))


def test_indexer_mask_long_rows(v41):
    """5000 tokens at ratio 1: the last tokens' wavefronts own more than 64
    key blocks each, so their live-block lists are built 64 blocks at a time."""
    T, HI, DI, L, blk = 5000, 4, 32, 5000, 16
    say("indexer mask long rows", T)
    rng = np.random.default_rng(5)
    qI = bf16_of(rng.standard_normal((T, HI, DI)))
    kI = bf16_of(rng.standard_normal((1, L, DI)))
    w = rng.uniform(0, 1, (T, HI)).astype(np.float32)
    cand = (rng.uniform(size=(T, (L + blk - 1) // blk)) < 0.5).astype(np.uint8)
    toks = [0, 1, 17, 1023, 1024, 2999, 4095, 4998, 4999]
    got = run_indexer(v41, qI, kI, w, 0, 1, cand=cand, cand_block=blk)[toks]
    ora = O.indexer_scores(qI, kI[0], w, 0, 1, cand=cand, cand_block=blk, tokens=toks)
    assert_scores_close(got, ora, "long masked rows", operands=(qI, kI[0], w, toks))


def test_indexer_zero_keys_give_zero(v41):
    HI, DI, L = 64, 128, 96
    rng = np.random.default_rng(8)
    qI = bf16_of(rng.standard_normal((1, HI, DI)))
    kI = np.zeros((1, L, DI), dtype=np.uint16)
    w = np.full((1, HI), 1 / 64, dtype=np.float32)
    got = run_indexer(v41, qI, kI, w, 10 ** 6, 1)
    assert np.all(got == 0.0)


# ------------------------------------------------------------------ top-k
def run_topk(v41, s, k, offset):
    R, L = s.shape
    d_s = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(DEV)
    d_i = torch.full((R, k + 2), -9, dtype=torch.int32, device=DEV)
    v41.v41_topk_select(d_s, R, L, L, k, offset, d_i, k + 2)
    torch.cuda.synchronize()
    got = d_i.cpu().numpy()
    assert np.all(got[:, k:] == -9)
    return got[:, :k]


def tie_scores(rng, R, L):
    s = (np.round(rng.standard_normal((R, L)) * 4) / 4).astype(np.float32)
    s[rng.uniform(size=(R, L)) < 0.05] = -np.inf
    s[rng.uniform(size=(R, L)) < 0.02] = np.nan
    z = rng.uniform(size=(R, L)) < 0.05
    s[z] = np.where(rng.uniform(size=z.sum()) < 0.5, 0.0, -0.0)
    return s


@pytest.mark.parametrize("R,L,k,offset", [(1, 1, 1, 0), (3, 7, 4, 128), (5, 512, 512, 2048),
                                          (4, 1000, 512, 128), (2, 4096, 512, 128),
                                          (2, 5000, 100, 0), (2, 32768, 512, 128),
                                          (1, 40000, 2048, 7), (64, 8192, 512, 128),
                                          (8, 300, 2048, 3), (6, 512, 64, 128),
                                          (3, 500, 100, 7), (4, 64, 16, 0),
                                          (3, 20001, 512, 128), (2, 30722, 700, 5),
                                          (3, 6001, 512, 0), (2, 3999, 256, 1),
                                          (2, 32768, 1, 0), (2, 32768, 2048, 3),
                                          (2, 24576, 2048, 0)])
def test_topk_parity_ties(v41, R, L, k, offset):
    say("topk", R, L, k, offset)
    rng = np.random.default_rng(R * 7 + L)
    s = tie_scores(rng, R, L)
    got = run_topk(v41, s, k, offset)
    want = O.topk(s, k, offset)
    assert np.array_equal(got, want)


def test_topk_continuous_scores(v41):
    rng = np.random.default_rng(3)
    s = (rng.uniform(0, 4, (16, 32768))).astype(np.float32)
    got = run_topk(v41, s, 512, 128)
    assert np.array_equal(got, O.topk(s, 512, 128))


def test_topk_all_excluded_and_signed_zeros(v41):
    s = np.full((3, 600), -np.inf, dtype=np.float32)
    s[1, :] = np.nan
    s[2, ::2] = -0.0
    s[2, 1::2] = 0.0
    got = run_topk(v41, s, 512, 5)
    want = O.topk(s, 512, 5)
    assert np.array_equal(got, want)
    assert np.all(got[0] == -1) and np.all(got[1] == -1)
    assert got[2].tolist() == [5 + j for j in range(512)]


@pytest.mark.parametrize("L", [512, 1024])
def test_topk_all_equal_scores(v41, L):
    """Every score equal (one radix bin from the start): the lowest k
    positions, with short rows on the one-wavefront select."""
    s = np.full((3, L), 0.75, dtype=np.float32)
    s[1, ::3] = -np.inf
    got = run_topk(v41, s, 100, 128)
    assert np.array_equal(got, O.topk(s, 100, 128))


def test_topk_big_tie_group_straddles_k(v41):
    L, k = 32768, 512
    rng = np.random.default_rng(9)
    s = rng.uniform(0, 1, (2, L)).astype(np.float32)
    pos = rng.permutation(L)[:301]
    s[:, pos] = np.sort(s[0])[-400]
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


@pytest.mark.parametrize("L", [8192, 32768, 40000])
@pytest.mark.parametrize("layout", ["fallback", "single_key_bins", "whole_bin", "in_bin_passes",
                                    "zeros_tie"])
def test_topk_radix_layouts(v41, L, layout):
    """Rows shaped to stress the radix passes: 3000 keys packed 2^-20 apart
    between two extremes, a key range under 1024 values, a selection that
    ends exactly at the bottom of a digit bin, a threshold group of 1500 close
    keys that takes three 8-bit passes, and 32k equal zeros.  Rows of 40000
    scores take the select that re-reads the row from memory."""
    say("topk radix layouts", L, layout)
    rng = np.random.default_rng(L + len(layout))
    k = 512
    if layout == "fallback":
        s = np.full(L, -1e30, dtype=np.float32)
        s[rng.integers(0, L)] = 1e30
        pos = rng.permutation(L)[:3000]
        s[pos] = 1.0 + np.arange(3000, dtype=np.float32) * np.float32(2.0 ** -20)
    elif layout == "single_key_bins":
        s = (1.0 + rng.integers(0, 1000, L) * 2.0 ** -23).astype(np.float32)
    elif layout == "whole_bin":
        s = rng.uniform(0, 1, L).astype(np.float32)
        pos = rng.permutation(L)[:k]
        s[pos] = (100.0 + rng.uniform(0, 1, k)).astype(np.float32)
    elif layout == "in_bin_passes":
        s = np.full(L, -1e30, dtype=np.float32)
        s[rng.integers(0, L)] = 1e30
        pos = rng.permutation(L)[:1500]
        s[pos] = 1.0 + rng.permutation(1500).astype(np.float32) * np.float32(2.0 ** -20)
    else:
        s = np.zeros(L, dtype=np.float32)
        s[rng.uniform(size=L) < 0.5] = -0.0
        pos = rng.permutation(L)[:300]
        s[pos] = rng.uniform(0.1, 1, 300).astype(np.float32)
    s = s[None, :]
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


@pytest.mark.parametrize("L,kpt", [(2048, 8), (4096, 16), (8192, 8), (32768, 32)])
@pytest.mark.parametrize("layout", ["samples_high", "samples_low", "one_value", "random"])
def test_topk_sampled_threshold_paths(v41, L, kpt, layout):
    """Rows whose every kpt-th position (the first position of each thread's
    range) holds the largest scores, the smallest scores, or where all but a
    few scores are equal: the sampled threshold then misses the top k (full
    select), lets too many through (full select) or is the k-th score itself
    (direct); random rows take the candidate path.  Rows of 32768 sample;
    the shorter ones check the plain select on the same layouts."""
    say("topk sampled", L, kpt, layout)
    rng = np.random.default_rng(L + len(layout))
    R, k = 3, 512
    s = rng.uniform(1, 2, (R, L)).astype(np.float32)
    if layout == "samples_high":
        s[:, ::kpt] += 10.0
    elif layout == "samples_low":
        s[:, ::kpt] -= 10.0
    elif layout == "one_value":
        s[:] = 0.5
        s[:, rng.permutation(L)[:100]] = 3.0
        s[1, ::7] = -0.0
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


@pytest.mark.parametrize("n_nonneg", [512, 1000])
def test_topk_long_threshold_at_signed_zero(v41, n_nonneg):
    """32768-score rows whose sample (every 32nd position) puts the sampled
    threshold at the boundary between -0 and the negative scores: 36 samples
    at or above zero (the expected count for k = 512 plus its margin), one of
    them -0, the other samples tiny negatives down to -2^-125, the row's
    largest score 1.0, so the first 8-bit digit window starts exactly at -0's
    key.  With 512 scores at or above zero the threshold is the 512th key
    (direct output); with 1000, 600 of them +-0, the top 512 come from the
    candidates and end inside the zero tie group (ties to the lower
    position, -0 == +0)."""
    say("topk threshold at -0", n_nonneg)
    rng = np.random.default_rng(n_nonneg)
    L, k = 32768, 512
    s = -rng.uniform(1e-30, 1.0, L).astype(np.float32)
    samp = np.arange(0, L, 32)
    s[samp] = -(rng.integers(1, 1 << 20, samp.size) * np.float32(2.0 ** -149)).astype(np.float32)
    s[samp[0]] = np.float32(-(2.0 ** -125))
    top = rng.permutation(samp[1:])[:36]
    s[top[:10]] = 0.0
    s[top[10:16]] = -0.0
    s[top[16:]] = rng.uniform(0.1, 0.9, 20).astype(np.float32)
    others = rng.permutation(np.setdiff1d(np.arange(L), samp))[:n_nonneg - 36]
    n_zero = 0 if n_nonneg == 512 else 600
    s[others[:n_zero // 2]] = 0.0
    s[others[n_zero // 2:n_zero]] = -0.0
    s[others[n_zero:]] = rng.uniform(0.0, 0.9, others.size - n_zero).astype(np.float32)
    s[others[-1]] = 1.0
    assert int((s >= 0).sum()) == n_nonneg
    s = s[None, :]
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


@pytest.mark.parametrize("n_valid,k", [(600, 512), (300, 512), (5000, 2048), (0, 64)])
def test_topk_long_mostly_unselectable(v41, n_valid, k):
    """32768-score rows where all but n_valid scores are NaN or -inf: fewer
    valid samples than the sampled threshold needs (full select), fewer
    valid scores than k (every valid one, then -1), none at all."""
    say("topk long mostly unselectable", n_valid, k)
    rng = np.random.default_rng(n_valid + k)
    L = 32768
    s = np.where(rng.uniform(size=(2, L)) < 0.5, np.float32(np.nan), np.float32(-np.inf))
    for r in range(2):
        pos = rng.permutation(L)[:n_valid]
        s[r, pos] = rng.standard_normal(n_valid).astype(np.float32)
    s = s.astype(np.float32)
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


def test_topk_long_candidates_overflow_one_wavefront(v41):
    """A 32768-score row whose first 2048 positions (one wavefront's share of
    the row) hold the high scores: the sampled threshold leaves about 990
    candidates, under the 4096-slot buffer, but some 560 of them in that
    wavefront's 256-slot region, so the row takes the full select; the
    second row spreads the same high scores over the whole row (candidate
    select)."""
    say("topk candidates overflow one wavefront")
    rng = np.random.default_rng(77)
    L, k = 32768, 512
    s = rng.uniform(0, 1, (2, L)).astype(np.float32)
    s[0, :2048] = rng.uniform(0.95, 1.0, 2048).astype(np.float32)
    s[1, rng.permutation(L)[:2048]] = rng.uniform(0.95, 1.0, 2048).astype(np.float32)
    got = run_topk(v41, s, k, 128)
    assert np.array_equal(got, O.topk(s, k, 128))


# ------------------------------------------------------------------ attention
def run_attn(v41, q, rows_a, rows_b, idx, sink, scale, B, T, use_ws=True):
    """q [B*T, H, D]; rows_a [B, A, D]; rows_b [B, Lb, D] or None; idx [B*T, width]."""
    Q, H, D = q.shape
    A = rows_a.shape[1]
    Lb = rows_b.shape[1] if rows_b is not None else 0
    width = idx.shape[1]
    d_out = torch.zeros(Q, H, D, dtype=torch.int16, device=DEV)
    ws_bytes = v41.v41_sparse_attn_workspace_bytes(B, T, H, D, width) if use_ws else 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV) if ws_bytes else None
    v41.v41_sparse_attn_sink(up16(q), up16(rows_a), A, A * D,
                             up16(rows_b) if rows_b is not None else None, Lb, Lb * D,
                             torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV),
                             width, width, torch.from_numpy(sink).to(DEV), scale, B, T, H, D,
                             d_out, ws, ws_bytes)
    return down16(d_out)


def oracle_attn(q, rows_a, rows_b, idx, sink, scale, B, T):
    outs = []
    for b in range(B):
        outs.append(O.sparse_attn(q[b * T:(b + 1) * T], rows_a[b],
                                  rows_b[b] if rows_b is not None else None,
                                  idx[b * T:(b + 1) * T], sink, scale))
    return np.concatenate(outs)


@pytest.mark.parametrize("B,T,H,D,A,Lb,width,use_ws", [
    (1, 1, 64, 512, 128, 1024, 640, True),     # decode, split rows
    (1, 1, 64, 512, 128, 1024, 640, False),    # decode, no workspace
    (3, 1, 64, 512, 128, 700, 640, True),
    (1, 40, 64, 512, 40, 100, 168, True),      # prefill-like, many -1
    (1, 12, 4, 64, 12, 4, 10, True),           # the tiny layer
    (2, 3, 70, 128, 50, 60, 97, True),         # heads over two groups, ragged
    (1, 5, 16, 256, 33, 0, 33, True),          # no compressed rows
    (1, 2, 64, 512, 64, 200, 120, True),       # one round of 8 tiles per workgroup
    (2, 1, 40, 512, 128, 300, 640, True),      # one round per split, a partial head group
    (1, 200, 70, 512, 64, 100, 64, True),      # wide form at 512 dims, a 6-head second group
    (1, 1, 64, 512, 128, 4000, 2048, True),    # widest row: 16 splits of one round each
    (1, 1, 64, 512, 128, 3000, 1536, True),    # 12 splits: a full and a partial combine chunk
    (2, 1, 64, 512, 128, 3000, 2048, False),   # widest row unsplit: 16 tiles per wavefront
    (1, 256, 64, 64, 256, 3000, 2048, True),   # widest row in the wide form (compacted list)
])
def test_attn_parity(v41, B, T, H, D, A, Lb, width, use_ws):
    say("attn", B, T, H, D, A, Lb, width, use_ws)
    rng = np.random.default_rng(B * 100 + H + D)
    q = bf16_of(rng.standard_normal((B * T, H, D)))
    rows_a = bf16_of(rng.standard_normal((B, A, D)))
    rows_b = bf16_of(rng.standard_normal((B, Lb, D))) if Lb > 0 else None
    idx = rng.integers(-1, A + Lb, (B * T, width)).astype(np.int32)
    idx[rng.uniform(size=idx.shape) < 0.2] = -1
    idx[:, -1] = A + Lb + 5          # out of range: skipped
    sink = rng.standard_normal(H).astype(np.float32)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = run_attn(v41, q, rows_a, rows_b, idx, sink, scale, B, T, use_ws)
    want = oracle_attn(q, rows_a, rows_b, idx, sink, scale, B, T)
    assert_attn_close(got, want, f"B{B} T{T} H{H} D{D} w{width} ws{use_ws}")


def test_attn_all_absent_and_one_row(v41):
    H, D = 64, 512
    rng = np.random.default_rng(1)
    q = bf16_of(rng.standard_normal((2, H, D)))
    rows_a = bf16_of(rng.standard_normal((1, 8, D)))
    idx = np.full((2, 16), -1, dtype=np.int32)
    idx[1, 5] = 3
    sink = rng.standard_normal(H).astype(np.float32)
    got = run_attn(v41, q, rows_a, None, idx, sink, 0.0625, 1, 2)
    assert np.all(got[0] == 0)
    want = oracle_attn(q, rows_a, None, idx, sink, 0.0625, 1, 2)
    assert_attn_close(got, want, "one row")


@pytest.mark.parametrize("seed", range(4, 12))
@pytest.mark.parametrize("A", [300, 120, 1200])
def test_attn_large_logits(v41, A, seed):
    """Scores far from zero (logits of standard deviation about 16, rows up to
    about 16 in size) exercise the running max (no overflow) and the
    precision of the probabilities in PV; 300 rows take two rounds per split
    (wavefronts merged at the end), 120 one round, 1200 nine splits (the
    combine's running max across two chunks)."""
    H, D = 64, 512
    rng = np.random.default_rng(seed)
    q = bf16_of(rng.standard_normal((1, H, D)) * 4)
    rows_a = bf16_of(rng.standard_normal((1, A, D)) * 4)
    idx = rng.permutation(A)[None, :].astype(np.int32)
    sink = (rng.standard_normal(H) * 30).astype(np.float32)
    got = run_attn(v41, q, rows_a, None, idx, sink, 0.044194173, 1, 1)
    want = oracle_attn(q, rows_a, None, idx, sink, 0.044194173, 1, 1)
    r = assert_attn_close(got, want, f"large logits A={A} seed={seed}")
    assert r["frac_within_2ulp"] >= 0.999, r


@pytest.mark.parametrize("seed", [4, 5])
def test_attn_large_logits_wide(v41, seed):
    """The same stress on the wide form (256 queries, so one workgroup per
    query and 64 heads): 120 rows, a few of them dominant per head."""
    T, H, D, A = 256, 64, 512, 120
    rng = np.random.default_rng(100 + seed)
    q = bf16_of(rng.standard_normal((T, H, D)) * 4)
    rows_a = bf16_of(rng.standard_normal((1, A, D)) * 4)
    idx = np.stack([rng.permutation(A) for _ in range(T)]).astype(np.int32)
    idx[rng.uniform(size=idx.shape) < 0.3] = -1
    sink = (rng.standard_normal(H) * 30).astype(np.float32)
    got = run_attn(v41, q, rows_a, None, idx, sink, 0.044194173, 1, T)
    want = oracle_attn(q, rows_a, None, idx, sink, 0.044194173, 1, T)
    r = assert_attn_close(got, want, f"large logits wide seed={seed}")
    assert r["frac_within_2ulp"] >= 0.999, r
