"""Host logic of bench.py, on the CPU: the algorithmic bytes and flops that
every roofline divides by (written out here from the workload shapes: rows
gathered, keys streamed, scores written and read), the roofline arithmetic,
the parity report that compares the CPU leg's oracle results with a step's
outputs, and the refusal of more than one GPU."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest
import torch

import bench
from inputs import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode64_step_bytes_and_flops():
    k = bench.algorithmic(W.WORKLOADS["decode64"])
    B, L, width = 64, 8192, 128 + 512
    # indexer: every key row of every sequence (128 bf16), each query's
    # 64 x 128 bf16 qI and 64 f32 weights, one f32 score per position
    assert k["indexer_scores"]["bytes"] == B * L * 256 + B * 16384 + B * 256 + B * L * 4
    assert k["indexer_scores"]["flops"] == B * L * 2 * 64 * 128          # 8.59 G
    # top-k: the scores read, 512 int32 written per row
    assert k["topk_select"]["bytes"] == B * L * 4 + B * 512 * 4
    # attention: 640 gathered 1 KB rows per query, its idx row, q and out
    att = k["sparse_attn_sink"]
    assert att["bytes"] == B * width * 1024 + B * width * 4 + 2 * B * 64 * 1024
    assert att["bytes"] == 50_495_488
    assert att["flops"] == B * width * 4 * 64 * 512                      # 5.37 G
    total = sum(v["bytes"] for v in k.values())
    assert abs(total / 1e6 - 190.27) < 0.01


def test_decode16_and_decode1_step_bytes():
    k16 = bench.algorithmic(W.WORKLOADS["decode16"])
    assert k16["sparse_attn_sink"]["bytes"] == 16 * 640 * 1024 + 16 * 640 * 4 + 2 * 16 * 65536
    assert k16["indexer_scores"]["flops"] == 16 * 32768 * 2 * 64 * 128
    assert abs(sum(v["bytes"] for v in k16.values()) / 1e6 - 151.38) < 0.01
    k1 = bench.algorithmic(W.WORKLOADS["decode1"])
    assert k1["indexer_scores"]["flops"] == 1024 * 2 * 64 * 128           # 16.8 M
    assert k1["sparse_attn_sink"]["flops"] == 640 * 4 * 64 * 512          # 83.9 M
    assert abs(sum(v["bytes"] for v in k1.values()) / 1e6 - 1.081) < 0.001


def test_prefill_attention_counts_valid_entries_only():
    """Prefill flops follow the idx rows handed in: 4 H D per entry >= 0; the
    chunk rows and latent rows are each read once."""
    wl = W.WORKLOADS["prefill"]
    idx = np.full((wl.n_tokens, wl.width), -1, dtype=np.int32)
    idx[:, :3] = 0
    idx[5, 100] = 7
    k = bench.algorithmic(wl, host_idx=idx, valid_pairs=1000)
    assert k["sparse_attn_sink"]["flops"] == (3 * wl.n_tokens + 1) * 4 * 64 * 512
    rows = (wl.n_tokens + wl.n_rows) * 1024
    assert k["sparse_attn_sink"]["bytes"] == rows + wl.n_tokens * wl.width * 4 + \
        2 * wl.n_tokens * 64 * 1024
    assert k["indexer_scores"]["flops"] == 1000 * 2 * 64 * 128


def test_roofline_entry_arithmetic():
    work = {"k": {"bytes": 8_000_000, "flops": 2_500_000_000}}
    kt = {"mean": 10.0, "p50": 9.5, "p90": 11.0}
    hbm = bench.roofline_entry("k", work, kt, "hbm", ceilings={"hbm_GBs": 6400.0})
    assert hbm["achieved"] == 800.0 and hbm["unit"] == "GB/s"
    assert hbm["frac"] == pytest.approx(800.0 / 8000.0)
    assert hbm["frac_of_measured"] == pytest.approx(800.0 / 6400.0, abs=1e-4)
    mf = bench.roofline_entry("k", work, kt, "mfma")
    assert mf["achieved"] == 250.0 and mf["unit"] == "TFLOP/s"
    assert mf["frac"] == pytest.approx(0.1)
    assert mf["frac_of_measured"] is None


def bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_parity_report_counts_ulps_and_selection():
    wl = W.WORKLOADS["decode1"]
    rng = np.random.default_rng(0)
    o = bf16_bits(rng.standard_normal((64, 512)) * 0.05)
    idx = np.concatenate([np.arange(128), 128 + np.arange(512)]).astype(np.int32)
    oracle = {0: (idx.copy(), o.copy())}

    def buf(i, out):
        return types.SimpleNamespace(idx=torch.from_numpy(i[None]),
                                     out=torch.from_numpy(out[None].view(np.int16)))

    same = bench.parity_report(buf(idx, o), wl, oracle)
    assert same["selection_equal"] == "1 of 1" and same["max_ulp"] == 0.0
    assert same["frac_within_2ulp"] == 1.0 and same["fail"] == 0
    # three ulp off in one output: counted, but within the 1e-2 absolute leg
    o2 = o.copy()
    o2[3, 7] += 3
    r = bench.parity_report(buf(idx, o2), wl, oracle)
    assert r["max_ulp"] == 3.0 and r["fail"] == 0
    assert r["frac_within_2ulp"] == pytest.approx(1 - 1 / o.size, abs=1e-6)
    # the top-k part compared as a set: a permutation still agrees, another
    # row does not (and then the outputs are not compared)
    perm = idx.copy()
    perm[128:] = perm[128:][::-1]
    assert bench.parity_report(buf(perm, o), wl, oracle)["selection_equal"] == "1 of 1"
    other = idx.copy()
    other[-1] = 128 + 600
    r = bench.parity_report(buf(other, o), wl, oracle)
    assert r["selection_equal"] == "0 of 1" and "max_ulp" not in r
    assert bench.parity_report(buf(idx, o), wl, {}) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
