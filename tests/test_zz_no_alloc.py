"""v41_sparse_attn_sink_noalloc (the attention for callers that cannot
allocate: row-split partials in the library's static device array) against
v41_sparse_attn_sink with a caller's workspace, through the C ABI.  Two calls
in a row on the shared array, the second with a smaller input, each checked
to the attention tolerance (2 bf16 ulp or 1e-2 absolute) against the
workspace form's output on the same inputs."""
import math

import numpy as np
import pytest
import torch

from inputs import synth as S
from parity import assert_attn_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def up16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def down16(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def case(B, A, Lb, width, H, D, seed):
    rng = np.random.default_rng(seed)
    bf = lambda x: S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    q = bf(rng.standard_normal((B, H, D)))
    rows_a = bf(rng.standard_normal((B, A, D)))
    rows_b = bf(rng.standard_normal((B, Lb, D)))
    idx = rng.integers(0, A + Lb, (B, width)).astype(np.int32)
    idx[rng.uniform(size=idx.shape) < 0.1] = -1
    sink = rng.standard_normal(H).astype(np.float32)
    return dict(q=up16(q), rows_a=up16(rows_a), rows_b=up16(rows_b),
                idx=torch.from_numpy(idx).to(DEV), sink=torch.from_numpy(sink).to(DEV),
                B=B, A=A, Lb=Lb, width=width, H=H, D=D)


def run(v41, c, noalloc):
    B, H, D, A, Lb, width = c["B"], c["H"], c["D"], c["A"], c["Lb"], c["width"]
    out = torch.zeros(B, H, D, dtype=torch.int16, device=DEV)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    args = (c["q"], c["rows_a"], A, A * D, c["rows_b"], Lb, Lb * D, c["idx"], width, width,
            c["sink"], scale, B, 1, H, D, out)
    if noalloc:
        v41.v41_sparse_attn_sink_noalloc(*args)
    else:
        wsb = v41.v41_sparse_attn_workspace_bytes(B, 1, H, D, width)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
        v41.v41_sparse_attn_sink(*args, ws, wsb)
    return down16(out)


def test_noalloc_matches_workspace_form():
    from indexer_top_sink_amd import v41
    v41.load()
    # long-context decode shape (16 sequences, 640 rows each), then one
    # sequence at context 4096: both split their rows, so both use the array
    for name, c in (("16 x 640", case(16, 128, 8192, 640, 64, 512, 11)),
                    ("1 x 640", case(1, 128, 1024, 640, 64, 512, 12))):
        need = v41.v41_sparse_attn_workspace_bytes(c["B"], 1, c["H"], c["D"], c["width"])
        print(f"[case] noalloc {name}: {need} bytes of scratch", flush=True)
        assert 0 < need <= 32 << 20
        want = run(v41, c, noalloc=False)
        got = run(v41, c, noalloc=True)
        r = assert_attn_close(got, want, f"noalloc {name}")
        print(f"[noalloc] {name}: bit-identical {bool(np.array_equal(got, want))}", flush=True)
        assert r["frac_within_2ulp"] == 1.0
