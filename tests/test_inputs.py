"""The seeded input generator against the published SplitMix64 and
Box-Muller definitions (CPU only), and the workloads' shapes."""
import math

import numpy as np

from inputs import synth as S
from inputs import workloads as W

M64 = (1 << 64) - 1


def mix(z):
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9 & M64
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB & M64
    return z ^ (z >> 31)


def test_splitmix64_reference_value():
    # SplitMix64 from state 0: the first output is mix(GAMMA)
    assert mix(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF


def test_stream_uniform_normal_match_definition():
    seed, tag = 12345, 7
    s0 = mix((seed * 0xD1342543DE82EF95 + tag) & M64)
    ref = [mix((s0 + (i + 1) * 0x9E3779B97F4A7C15) & M64) for i in range(10)]
    assert [int(v) for v in S.stream_u64(seed, tag, 10)] == ref
    assert np.array_equal(S.uniform(seed, tag, 10), [(r >> 11) * 2.0 ** -53 for r in ref])
    n = S.normal(seed, tag, 6)
    for p in range(3):
        u1 = 1 - (ref[2 * p] >> 11) * 2.0 ** -53
        u2 = (ref[2 * p + 1] >> 11) * 2.0 ** -53
        r = math.sqrt(-2 * math.log(u1))
        assert abs(n[2 * p] - r * math.cos(2 * math.pi * u2)) < 1e-15
        assert abs(n[2 * p + 1] - r * math.sin(2 * math.pi * u2)) < 1e-15


def test_parallel_blocks_equal_serial_and_slices():
    n = (1 << 21) + 12345
    a = S.normal(3, 4, n)
    b = S.normal(3, 4, 1000)
    assert np.array_equal(a[:1000], b)
    u = S.uniform(3, 5, n)
    assert np.array_equal(u[(1 << 20) - 3:(1 << 20) + 3], S.uniform(3, 5, 6, start=(1 << 20) - 3))
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)
    assert S.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_workload_shapes():
    wl = W.WORKLOADS["decode64"]
    assert (wl.batch, wl.n_rows, wl.width, wl.rows_a_len) == (64, 8192, 640, 128)
    assert (wl.start_pos + 1) // wl.ratio == wl.n_rows
    p = W.WORKLOADS["prefill"]
    assert (p.n_tokens, p.width, p.rows_a_len, p.cand_width * p.cand_block) == (2048, 640, 2048, 512)
    assert W.WORKLOADS["decode16"].n_rows == (131071 + 1) // 4
    assert W.WORKLOADS["decode1"].n_rows == (4095 + 1) // 4
    t = W.TINY
    assert (t.width, t.n_rows) == (10, 4)
    assert len(W.tie_source_rows()) == 8
