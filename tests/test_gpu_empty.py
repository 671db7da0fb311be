"""Degenerate sizes through the C ABI: calls with nothing to do return
success and leave every buffer as it was; a top-k row with no columns is all
-1 padding; attention over an empty selection gives O = 0 (the sink alone
fills the denominator), in the narrow, wide and no-allocation entry points.
Expected values come from the oracle on the same empty shapes."""
import numpy as np
import pytest
import torch

import oracle as O
from inputs import synth as S

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def v41():
    from indexer_top_sink_amd import v41 as m
    m.load()
    return m


def say(*a):
    print("[case]", *a, flush=True)


def test_zero_sized_calls_touch_nothing(v41):
    """Each of the five calls with zero rows, sequences or queries: status 0,
    and the buffers it was handed keep their sentinel."""
    say("zero-sized calls")
    D = 512
    buf16 = torch.full((4, D), 1234, dtype=torch.int16, device=DEV)
    ring = torch.full((8, D), 77, dtype=torch.int16, device=DEV)
    v41.v41_fp8_round_rows(None, D, None, D, 0, D)
    v41.v41_fp8_round_rows(buf16, D, buf16, D, 0, D, ring, 8, 5)
    idx = torch.full((2, 16), -9, dtype=torch.int32, device=DEV)
    assert v41.v41_window_idx(40, 1, 8, 0, idx, 16, 16) == 8
    assert v41.v41_window_idx(0, 0, 8, 2, idx, 16, 16) == 0
    scores = torch.full((2, 4), 7.0, dtype=torch.float32, device=DEV)
    qI = torch.zeros((2, 64, 128), dtype=torch.int16, device=DEV)
    w = torch.zeros((2, 64), dtype=torch.float32, device=DEV)
    v41.v41_indexer_scores(None, None, 0, None, None, 0, 1, 0, 1, 100, 4, 64, 128, 32, None, 32)
    # two decode queries, no compressed rows published yet: nothing to score
    v41.v41_indexer_scores(qI, qI, 0, w, None, 0, 1, 2, 1, 100, 4, 64, 128, 0, scores, 4)
    v41.v41_topk_select(None, 0, 100, 100, 16, 0, None, 16)
    v41.v41_sparse_attn_sink(None, None, 0, 0, None, 0, 0, None, 16, 16, None, 0.1, 0, 1, 64,
                             D, None)
    v41.v41_sparse_attn_sink_noalloc(None, None, 0, 0, None, 0, 0, None, 16, 16, None, 0.1, 0,
                                     1, 64, D, None)
    torch.cuda.synchronize()
    assert torch.all(buf16 == 1234) and torch.all(ring == 77)
    assert torch.all(idx == -9)
    assert torch.all(scores == 7.0)


def test_topk_rows_without_columns(v41):
    """No scores in a row (n_cols = 0, no score buffer): k entries of -1."""
    say("topk with no columns")
    R, k = 3, 5
    d_i = torch.full((R, k + 2), -9, dtype=torch.int32, device=DEV)
    v41.v41_topk_select(None, R, 0, 0, k, 7, d_i, k + 2)
    torch.cuda.synchronize()
    got = d_i.cpu().numpy()
    assert np.array_equal(got[:, :k], O.topk(np.zeros((R, 0), np.float32), k, 7))
    assert np.all(got[:, k:] == -9)


@pytest.mark.parametrize("B,T,H,D", [(3, 1, 64, 512), (1, 300, 64, 512), (2, 1, 20, 128)])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_attn_empty_selection_gives_zero(v41, B, T, H, D, entry):
    """width = 0 (no idx buffer): every output row is 0, as the oracle's
    sink-only softmax gives, in the narrow (few queries) and the wide (300
    queries) forms."""
    say("attention width 0", B, T, H, D, entry)
    rng = np.random.default_rng(5)
    Q = B * T
    q = S.f32_to_bf16_bits(rng.standard_normal((Q, H, D)).astype(np.float32))
    rows = S.f32_to_bf16_bits(rng.standard_normal((B, 4, D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    d_q = torch.from_numpy(q.view(np.int16)).to(DEV)
    d_rows = torch.from_numpy(rows.view(np.int16)).to(DEV)
    d_sink = torch.from_numpy(sink).to(DEV)
    d_out = torch.full((Q, H, D), 1234, dtype=torch.int16, device=DEV)
    scale = 1.0 / np.sqrt(D)
    if entry == "workspace":
        assert v41.v41_sparse_attn_workspace_bytes(B, T, H, D, 0) == 0
        v41.v41_sparse_attn_sink(d_q, d_rows, 4, 4 * D, None, 0, 0, None, 0, 0, d_sink, scale,
                                 B, T, H, D, d_out)
    else:
        v41.v41_sparse_attn_sink_noalloc(d_q, d_rows, 4, 4 * D, None, 0, 0, None, 0, 0, d_sink,
                                         scale, B, T, H, D, d_out)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint16)
    want = np.concatenate([O.sparse_attn(q[b * T:(b + 1) * T], rows[b], None,
                                         np.zeros((T, 0), np.int32), sink, scale)
                           for b in range(B)])
    assert np.array_equal(got, want)
