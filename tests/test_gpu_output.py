"""GPU parity of the bf16 projections (v41_linear_bf16) and the grouped output
projection (v41_grouped_output) against the oracle.

The GPU accumulates in f32 (and, at decode sizes, adds per-split f32 partial
sums), the oracle in double with one rounding, so an output may differ by one
bf16 ulp where the two sides straddle a rounding boundary, plus the f32
accumulation error: |gpu - oracle| <= ulp_bf16(oracle) + 2^-14 * sum_k
|a_k w_k| (the second term is far above the f32 error of these sums and far
below a bf16 ulp of typical outputs)."""
import numpy as np
import pytest
import torch

import oracle as O
from inputs import synth as S

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def v41():
    from indexer_top_sink_amd import v41 as m
    m.load()
    return m


def say(*a):
    print("[case]", *a, flush=True)


def up16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def down16(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def f64(h):
    return S.bf16_bits_to_f32(np.asarray(h, dtype=np.uint16)).astype(np.float64)


def ulp_bf16(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_linear_close(got, want, a, w, what):
    g, o = f64(got), f64(want)
    bound = ulp_bf16(o) + 2.0 ** -14 * (np.abs(f64(a)) @ np.abs(f64(w)).T)
    err = np.abs(g - o)
    exact = float((err == 0).mean())
    print(f"[linear parity] {what} exact={exact:.4f} max_ulp={float((err / ulp_bf16(o)).max()):.2f}",
          flush=True)
    assert np.all(err <= bound), what


def weights(seed, shape, fan_in):
    """N(0, 1/fan_in) bf16 weights (synthetic: no trained weights exist here)."""
    x = S.normal_f32(seed, S.TAG_MISC, shape) * np.float32(1.0 / np.sqrt(fan_in))
    return S.f32_to_bf16_bits(x)


@pytest.mark.parametrize("M,N,K,G,sample", [
    (64, 1024, 4096, 8, 8),       # wo_a at a 64-token decode
    (64, 5120, 8192, 1, 6),       # wo_b at a 64-token decode
    (300, 200, 192, 1, None),     # ragged rows and columns, large-tile path
    (17, 72, 128, 3, None),       # ragged, grouped, small-tile path
    (2048, 512, 1024, 1, 24),     # many rows
    (1, 64, 64, 1, None),
    (5, 70, 2048, 2, None),       # split K with N not a multiple of 4
])
def test_linear_parity(v41, M, N, K, G, sample):
    say("linear", M, N, K, G)
    a = S.normal_bf16(100 + M, S.TAG_Q, (M, G * K))           # groups side by side
    w = weights(200 + N, (G * N, K), K)
    d_a, d_w = up16(a), up16(w)
    ws_bytes = v41.v41_linear_workspace_bytes(M, N, K, G)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    for use_ws in (True, False):
        d_y = torch.full((M, G * N), 0x1234, dtype=torch.int16, device=DEV)
        v41.v41_linear_bf16(d_a, G * K, K, d_w, K, N * K, d_y, G * N, N, M, N, K, G,
                            ws if use_ws else None, ws_bytes if use_ws else 0)
        y = down16(d_y)
        rows = np.arange(M) if sample is None else np.linspace(0, M - 1, sample).astype(int)
        for g in range(G):
            ag = a[rows][:, g * K:(g + 1) * K]
            wg = w[g * N:(g + 1) * N]
            assert_linear_close(y[rows][:, g * N:(g + 1) * N], O.linear_bf16(ag, wg), ag, wg,
                                f"M={M} N={N} K={K} g={g} ws={use_ws}")


def test_linear_no_rows(v41):
    v41.v41_linear_bf16(None, 64, 0, None, 64, 0, None, 64, 0, 0, 64, 64, 1)
    torch.cuda.synchronize()


def test_grouped_output_decode64():
    """The output side of a 64-token decode step: o (64 heads x 512) through
    the inverse rotation at position 32767, then wo_a (8 groups, rank 1024)
    and wo_b (dim 5120), synthetic weights."""
    from indexer_top_sink_amd import layer as LY
    from indexer_top_sink_amd import v41
    T, H, D, G, R, dim, rd, p = 64, 64, 512, 8, 1024, 5120, 64, 32767
    gw = H * D // G
    say("grouped output decode64")
    o = S.normal_bf16(301, S.TAG_Q, (T, H, D))
    wa = weights(302, (G * R, gw), gw)
    wb = weights(303, (dim, G * R), G * R)
    rt = LY.rope_table(10000.0, rd, p + 1, DEV)
    d_o = up16(o)
    v41.v41_rope_rows(d_o, D, d_o, D, T, 1, H, D, rd, rt.table, rt.n_pos, None, p, 1)
    o_bar = down16(d_o)
    tab = O.rope_table(10000.0, rd, p + 1)
    assert np.array_equal(o_bar.reshape(T * H, D),
                          O.rope_rows(o.reshape(T * H, D), tab, np.full(T * H, p), rd,
                                      inverse=True))
    d_og = torch.empty(T, G * R, dtype=torch.int16, device=DEV)
    d_x = torch.empty(T, dim, dtype=torch.int16, device=DEV)
    wsb = v41.v41_grouped_output_workspace_bytes(T, H, D, G, R, dim)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    d_wa, d_wb = up16(wa), up16(wb)
    v41.v41_grouped_output(d_o, T, H, D, G, R, dim, d_wa, d_wb, d_og, d_x, workspace=ws,
                           workspace_bytes=wsb)
    og, x = down16(d_og), down16(d_x)
    # the inverse rotation requested from the call, on the unrotated o: the
    # same bits as rotating first (positions from a device array)
    d_o2 = up16(o)
    d_og2 = torch.empty_like(d_og)
    d_x2 = torch.empty_like(d_x)
    pos = torch.full((T,), p, dtype=torch.int32, device=DEV)
    v41.v41_grouped_output(d_o2, T, H, D, G, R, dim, d_wa, d_wb, d_og2, d_x2, rope_table=rt.table,
                           rope_rows=rt.n_pos, rope_dim=rd, pos=pos, workspace=ws,
                           workspace_bytes=wsb)
    assert np.array_equal(down16(d_og2), og)
    assert np.array_equal(down16(d_x2), x)
    assert np.array_equal(down16(d_o2), o_bar)  # o's tails rotated back in place
    rows = [0, 21, 42, 63]
    ob = o_bar.reshape(T, H * D)[rows]
    for g in range(G):
        ag = ob[:, g * gw:(g + 1) * gw]
        wg = wa[g * R:(g + 1) * R]
        assert_linear_close(og[rows][:, g * R:(g + 1) * R], O.linear_bf16(ag, wg), ag, wg,
                            f"og group {g}")
    # wo_b on the GPU's own (checked) og
    assert_linear_close(x[rows], O.linear_bf16(og[rows], wb), og[rows], wb, "x")


def test_grouped_output_prefill_with_rotation():
    """2048 tokens at positions 0.., the inverse rotation requested from the
    call against rotating first; sampled rows against the oracle."""
    from indexer_top_sink_amd import layer as LY
    from indexer_top_sink_amd import v41
    T, H, D, G, R, dim, rd = 2048, 64, 512, 8, 1024, 640, 64
    gw = H * D // G
    say("grouped output prefill, with the inverse rotation")
    o = S.normal_bf16(311, S.TAG_Q, (T, H, D))
    wa = weights(312, (G * R, gw), gw)
    wb = weights(313, (dim, G * R), G * R)
    rt = LY.rope_table(10000.0, rd, T, DEV)
    d_wa, d_wb = up16(wa), up16(wb)
    d_og = torch.empty(T, G * R, dtype=torch.int16, device=DEV)
    d_x = torch.empty(T, dim, dtype=torch.int16, device=DEV)
    d_o = up16(o)
    v41.v41_grouped_output(d_o, T, H, D, G, R, dim, d_wa, d_wb, d_og, d_x, rope_table=rt.table,
                           rope_rows=rt.n_pos, rope_dim=rd, start_pos=0)
    og, x = down16(d_og), down16(d_x)
    d_o = up16(o)
    v41.v41_rope_rows(d_o, D, d_o, D, 1, T, H, D, rd, rt.table, rt.n_pos, None, 0, 1)
    d_og2 = torch.empty_like(d_og)
    d_x2 = torch.empty_like(d_x)
    v41.v41_grouped_output(d_o, T, H, D, G, R, dim, d_wa, d_wb, d_og2, d_x2)
    assert np.array_equal(down16(d_og2), og)
    assert np.array_equal(down16(d_x2), x)
    o_bar = down16(d_o).reshape(T, H * D)
    rows = [0, 1, 1000, 2047]
    for g in (0, 5):
        ag = o_bar[rows][:, g * gw:(g + 1) * gw]
        wg = wa[g * R:(g + 1) * R]
        assert_linear_close(og[rows][:, g * R:(g + 1) * R], O.linear_bf16(ag, wg), ag, wg,
                            f"prefill og group {g}")
    assert_linear_close(x[rows], O.linear_bf16(og[rows], wb), og[rows], wb, "prefill x")
