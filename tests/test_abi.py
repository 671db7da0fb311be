"""The C ABI without a GPU: libv41.so loads, exports every entry point that
include/v41.h declares, and rejects invalid arguments on the host (these
calls return before any device work, so they run on the CPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "v41.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(v41_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from indexer_top_sink_amd import v41
    if not os.path.exists(v41.LIB_PATH):
        pytest.fail("libv41.so is not built (python -m indexer_top_sink_amd.build)")
    return v41.load()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("v41_fp8_round_rows", "v41_window_idx", "v41_indexer_scores",
              "v41_topk_select", "v41_sparse_attn_sink"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from indexer_top_sink_amd import v41
    assert set(v41.EXPORTS) == set(declared_functions())


def test_abi_version(lib):
    assert lib.v41_abi_version() == 8


def _err(lib):
    return lib.v41_last_error().decode()


def test_fp8_rejects_bad_row_len(lib):
    rc = lib.v41_fp8_round_rows(None, 48, None, 48, 1, 48, None, 0, 0, None)
    assert rc == -1 and "row_len" in _err(lib)


def test_fp8_rejects_unaligned(lib):
    rc = lib.v41_fp8_round_rows(16 + 2, 64, 32, 64, 1, 64, None, 0, 0, None)
    assert rc == -1 and "aligned" in _err(lib)


def test_window_rejects_multi_token_decode(lib):
    cols = C.c_int32(0)
    rc = lib.v41_window_idx(5, 2, 8, 1, 1024, 8, 16, C.byref(cols), None)
    assert rc == -1 and "one token" in _err(lib)


def test_indexer_rejects_missing_cache(lib):
    rc = lib.v41_indexer_scores(1024, None, 0, 1024, None, 0, 1, 1, 1, 100, 4, 64, 128, 10,
                                1024, 10, None)
    assert rc == -1 and "kI NULL" in _err(lib)


def test_indexer_rejects_ratio_and_heads(lib):
    assert lib.v41_indexer_scores(1024, 1024, 0, 1024, None, 0, 1, 1, 1, 100, 0, 64, 128, 10,
                                  1024, 10, None) == -1
    assert "ratio" in _err(lib)
    assert lib.v41_indexer_scores(1024, 1024, 0, 1024, None, 0, 1, 1, 1, 100, 4, 65, 128, 10,
                                  1024, 10, None) == -1
    assert lib.v41_indexer_scores(1024, 1024, 0, 1024, None, 0, 1, 1, 1, 100, 4, 64, 96, 10,
                                  1024, 10, None) == -1


def test_topk_rejects_k(lib):
    assert lib.v41_topk_select(1024, 1, 10, 10, 0, 0, 1024, 10, None) == -1
    assert lib.v41_topk_select(1024, 1, 10, 10, 2049, 0, 1024, 4096, None) == -1


def test_attn_rejects_wide_selection_and_missing_rows(lib):
    rc = lib.v41_sparse_attn_sink(1024, 1024, 128, 0, 1024, 10, 0, 1024, 2049, 4096, 1024,
                                  C.c_float(0.1), 1, 1, 64, 512, 1024, None, 0, None)
    assert rc == -1 and "width" in _err(lib)
    rc = lib.v41_sparse_attn_sink(1024, 1024, 128, 0, None, 10, 0, 1024, 640, 640, 1024,
                                  C.c_float(0.1), 1, 1, 64, 512, 1024, None, 0, None)
    assert rc == -1 and "rows_b" in _err(lib)
    rc = lib.v41_sparse_attn_sink(1024, 1024, 128, 0, None, 0, 0, 1024, 640, 640, 1024,
                                  C.c_float(0.1), 1, 1, 64, 320, 1024, None, 0, None)
    assert rc == -1 and "head_dim" in _err(lib)


def test_workspace_query(lib):
    # few queries: the call would split rows and asks for scratch; the size
    # holds an f32 partial O and (max, sum) per (query, split, head)
    ws = lib.v41_sparse_attn_workspace_bytes(16, 1, 64, 512, 640)
    assert ws > 0 and ws % (16 * 64 * (512 * 4 + 8)) == 0
    # 64 queries x 4 groups of 16 heads already cover the compute units
    assert lib.v41_sparse_attn_workspace_bytes(64, 1, 64, 512, 640) == 0
    # many queries: no split
    assert lib.v41_sparse_attn_workspace_bytes(1, 2048, 64, 512, 640) == 0


def test_rope_table_rejects_odd_dim_and_theta(lib):
    assert lib.v41_rope_table(10000.0, 63, 4, 1024, None) == -1 and "even" in _err(lib)
    assert lib.v41_rope_table(0.0, 64, 4, 1024, None) == -1 and "theta" in _err(lib)
    assert lib.v41_rope_table(10000.0, 64, 4, 1028, None) == -1 and "aligned" in _err(lib)


def test_rope_rows_rejects_bad_shapes(lib):
    # rope_dim not a multiple of 8
    assert lib.v41_rope_rows(1024, 64, 1024, 64, 1, 1, 1, 64, 12, 4096, 10, None, 0, 0,
                             None) == -1 and "rope_dim" in _err(lib)
    # rope_dim wider than the row
    assert lib.v41_rope_rows(1024, 64, 1024, 64, 1, 1, 1, 64, 72, 4096, 10, None, 0, 0,
                             None) == -1
    # host positions past the table
    assert lib.v41_rope_rows(1024, 64, 1024, 64, 1, 4, 1, 64, 16, 4096, 10, None, 7, 0,
                             None) == -1 and "outside the table" in _err(lib)
    # distinct but overlapping in and out
    assert lib.v41_rope_rows(1 << 20, 64, (1 << 20) + 16, 64, 1, 4, 1, 64, 16, 4096, 10, None,
                             0, 0, None) == -1 and "overlap" in _err(lib)
    # in place with different strides
    assert lib.v41_rope_rows(1 << 20, 64, 1 << 20, 72, 1, 4, 1, 64, 16, 4096, 10, None, 0, 0,
                             None) == -1


def test_rope_fp8_rows_rejects_bad_shapes(lib):
    # row_len not a multiple of the fp8 block
    assert lib.v41_rope_fp8_rows(1024, 48, 4096, 48, 1, 1, 48, 16, 8192, 10, None, 0, None, 0,
                                 0, None) == -1 and "row_len" in _err(lib)
    # nowhere to write
    assert lib.v41_rope_fp8_rows(1024, 64, None, 64, 1, 1, 64, 16, 8192, 10, None, 0, None, 0,
                                 0, None) == -1 and "neither" in _err(lib)
    # ring too small for the batch stride
    assert lib.v41_rope_fp8_rows(1 << 20, 64, None, 64, 2, 1, 64, 16, 8192, 10, None, 0,
                                 1 << 24, 8, 64, None) == -1 and "ring_bs" in _err(lib)
    # ring overlapping the input rows
    assert lib.v41_rope_fp8_rows(1 << 20, 64, None, 64, 1, 4, 64, 16, 8192, 10, None, 0,
                                 (1 << 20) + 256, 8, 512, None) == -1 and "overlaps" in _err(lib)


def test_decode_step_args_layout_matches_header(tmp_path):
    """The ctypes mirror of v41_decode_step_args has the C compiler's size and
    field offsets (a small C program built against include/v41.h prints them)."""
    import ctypes
    import subprocess

    from indexer_top_sink_amd import v41
    fields = [f for f, _ in v41.DecodeStepArgs._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "v41.h"', "int main(void) {",
           '  printf("%zu\\n", sizeof(v41_decode_step_args));']
    src += [f'  printf("%zu\\n", offsetof(v41_decode_step_args, {f}));' for f in fields]
    src += ["  return 0;", "}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(c), "-o",
                    str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(v41.DecodeStepArgs)
    for f, off in zip(fields, got[1:]):
        assert getattr(v41.DecodeStepArgs, f).offset == off, f


def _step_args(**over):
    from indexer_top_sink_amd import v41
    base = dict(batch=2, n_heads=64, head_dim=512, window=128, ratio=4, index_heads=64,
                index_dim=128, topk=512, rope_dim=0, scale=0.04, n_rows=1024, rope_rows=0,
                ring_bs=128 * 512, latent_bs=1024 * 512, kI_bs=1024 * 128, workspace_bytes=0,
                pos=1 << 20, q=2 << 20, kv_new=3 << 20, ring=4 << 20, latent=5 << 20,
                kI=6 << 20, qI=7 << 20, w=8 << 20, rope_table=None, sink=9 << 20,
                scores=10 << 20, idx=11 << 20, out=12 << 20, workspace=None)
    base.update(over)
    return v41.DecodeStepArgs.make(**base)


def test_decode_step_rejects_bad_arguments(lib):
    import ctypes
    cases = [
        (dict(pos=None), "NULL pos"),
        (dict(head_dim=320), "head_dim"),
        (dict(topk=2000), "selection limit"),
        (dict(rope_dim=64), "rope_table"),
        (dict(rope_dim=12, rope_table=13 << 20, rope_rows=10), "rope_dim"),
        (dict(ring_bs=100), "ring_bs"),
        (dict(latent=None), "no latent cache"),
        (dict(index_dim=96), "index_dim"),
        (dict(q=(2 << 20) + 4), "aligned"),
    ]
    for over, msg in cases:
        a = _step_args(**over)
        rc = lib.v41_decode_step(ctypes.byref(a), None)
        assert rc == -1 and msg in _err(lib), (over, _err(lib))
    assert lib.v41_decode_step(None, None) == -1


def test_candidate_blocks_rejects_bad_arguments(lib):
    assert lib.v41_candidate_blocks(1024, 1, 64, 64, 0, 4, 4096, 8, None) == -1
    assert "cand_block" in _err(lib)
    assert lib.v41_candidate_blocks(1024, 1, 64, 64, 8, 0, 4096, 8, None) == -1
    assert lib.v41_candidate_blocks(1024, 1, 64, 64, 8, 4, 4096, 7, None) == -1
    assert "cand_ld" in _err(lib)
    assert lib.v41_candidate_blocks(1024, 1, 1 << 20, 1 << 20, 8, 4, 4096, 1 << 17,
                                    None) == -1 and "exceed" in _err(lib)


def test_linear_rejects_bad_arguments(lib):
    assert lib.v41_linear_bf16(1024, 96, 0, 4096, 96, 0, 8192, 8, 0, 4, 8, 96, 1, None, 0,
                               None) == -1 and "multiple of 64" in _err(lib)
    assert lib.v41_linear_bf16(1024, 60, 0, 4096, 64, 0, 8192, 8, 0, 4, 8, 64, 1, None, 0,
                               None) == -1 and "lda" in _err(lib)
    assert lib.v41_linear_bf16(1028, 64, 0, 4096, 64, 0, 8192, 8, 0, 4, 8, 64, 1, None, 0,
                               None) == -1 and "aligned" in _err(lib)
    assert lib.v41_grouped_output(1024, 4, 6, 64, 4, 64, 64, 4096, 8192, 16384, 32768, None, 0,
                                  0, None, 0, None, 0, None) == -1
    assert "multiple of groups" in _err(lib)
    # rotation requested with a rope_dim that is not a multiple of 8
    assert lib.v41_grouped_output(1024, 4, 8, 64, 4, 64, 64, 4096, 8192, 16384, 32768, 65536, 10,
                                  12, None, 0, None, 0, None) == -1 and "rope_dim" in _err(lib)


def test_workspace_queries_for_projections(lib):
    # decode sizes split K (f32 partials per split); prefill sizes do not
    assert lib.v41_linear_workspace_bytes(64, 5120, 8192, 1) > 0
    assert lib.v41_linear_workspace_bytes(2048, 5120, 8192, 1) == 0
    assert lib.v41_grouped_output_workspace_bytes(64, 64, 512, 8, 1024, 5120) > 0
