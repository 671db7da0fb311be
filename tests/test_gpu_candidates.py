"""GPU parity of the candidate-block selection (v41_candidate_blocks) against
the oracle: bit-exact masks on the same f32 scores (ties, -inf, NaN, +-0,
every launch shape up to the block limit), and the chain that uses it -- a
candidate source's indexer scores, its block mask, and an index source's
indexer scores under that mask."""
import numpy as np
import pytest
import torch

import oracle as O
from inputs import synth as S
from inputs import workloads as W
from parity import assert_scores_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def v41():
    from indexer_top_sink_amd import v41 as m
    m.load()
    return m


def say(*a):
    print("[case]", *a, flush=True)


def tricky_scores(seed, R, L):
    """Rows with many equal values across blocks, -inf runs, NaN and +-0."""
    u = S.uniform(seed, S.TAG_MISC, R * L).reshape(R, L)
    z = S.normal(seed, S.TAG_TIES, R * L).reshape(R, L)
    s = np.where(u < 0.5, np.round(z * 4) / 4, z).astype(np.float32)
    s[u > 0.9] = -np.inf
    s[(u > 0.88) & (u <= 0.885)] = np.nan
    s[(u > 0.2) & (u <= 0.21)] = -0.0
    s[:, L - L // 5:] = -np.inf          # a causal tail
    return s


@pytest.mark.parametrize("R,L,cb,k", [(5, 200, 4, 7), (2, 13, 5, 1), (3, 1000, 8, 2048),
                                      (64, 8192, 8, 512), (16, 32768, 8, 2048),
                                      (2, 131072, 8, 2048), (1, 262144, 8, 2048),
                                      (4, 5000, 1, 300), (3, 1003, 8, 100)])
def test_candidate_blocks_parity(v41, R, L, cb, k):
    say("candidate blocks", R, L, cb, k)
    s = tricky_scores(1000 + L, R, L)
    nb = -(-L // cb)
    d_s = torch.from_numpy(s).to(DEV)
    ld = nb + 3
    d_c = torch.full((R, ld), 7, dtype=torch.uint8, device=DEV)
    v41.v41_candidate_blocks(d_s, R, L, L, cb, k, d_c, ld)
    torch.cuda.synchronize()
    got = d_c.cpu().numpy()
    want = O.candidate_blocks(s, cb, k)
    assert np.array_equal(got[:, :nb], want)
    assert np.all(got[:, nb:] == 7)


def test_candidate_chain_decode16():
    """A candidate source over decode16's sequences: its indexer scores, the
    top 2048 of 4096 blocks of 8, then an index source's scores under that
    mask (another query, the same index keys)."""
    from bench import stage_decode
    from indexer_top_sink_amd import v41
    wl = W.WORKLOADS["decode16"]
    say("candidate chain decode16")
    buf, host = stage_decode(wl, DEV, keep_host=True)
    B, L, HI, DI = wl.batch, wl.n_rows, wl.index_heads, wl.index_dim
    v41.v41_indexer_scores(buf.qI, buf.kI, L * DI, buf.w, None, 0, 1, B, 1, wl.start_pos,
                           wl.ratio, HI, DI, L, buf.scores, L)
    cb, kb = 8, 2048
    nb = L // cb
    cand = torch.zeros(B, nb, dtype=torch.uint8, device=DEV)
    v41.v41_candidate_blocks(buf.scores, B, L, L, cb, kb, cand, nb)
    torch.cuda.synchronize()
    scores = buf.scores.cpu().numpy()
    mask = cand.cpu().numpy()
    assert np.array_equal(mask, O.candidate_blocks(scores, cb, kb))
    assert np.all(mask.sum(axis=1) == kb)
    # an index source with its own queries under the candidate mask
    qI2 = S.normal_bf16(4242, S.TAG_QI, (B, HI, DI))
    from indexer_top_sink_amd import layer as LY
    buf.qI.copy_(LY.to_device_bf16(qI2, DEV))
    scores2 = torch.empty(B, L, dtype=torch.float32, device=DEV)
    v41.v41_indexer_scores(buf.qI, buf.kI, L * DI, buf.w, cand, nb, cb, B, 1, wl.start_pos,
                           wl.ratio, HI, DI, L, scores2, L)
    torch.cuda.synchronize()
    g2 = scores2.cpu().numpy()
    blocked = np.repeat(mask == 0, cb, axis=1)
    assert np.all(np.isneginf(g2[blocked]))
    for b in (0, 9, 15):
        ora = O.indexer_scores(qI2[b:b + 1], host[b]["kI"], host[b]["w"], wl.start_pos, wl.ratio,
                               cand=mask[b:b + 1], cand_block=cb)
        assert_scores_close(g2[b:b + 1], ora, f"masked scores b={b}")
