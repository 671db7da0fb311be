"""Pins of the oracle's rotary embedding (CPU only).

What fixes the expected values: the apply_rotary and freqs_cis contracts and
the precision paragraph of the "deepseek_v41_ref::attn" rustdoc (the last
rope_dim values of a row, adjacent pairs as complex numbers, binary32
products, bf16 results, the negated angle for the inverse; a [seqlen][dim/2]
table of (cos, sin) without YaRN), the rotations R_t and R_t^-1 of the "All
25 steps" section of the "Compressed sparse attention" layer page and the
config on that page (rope_head_dim 64, rope_theta 10000).  The frequency
ladder theta^(-2i/dim) is a reading; the hand table values pin it.
"""
import math

import numpy as np
import pytest

import oracle as O
from golden_io import kv, lines, num

from inputs import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(h):
    return synth.bf16_bits_to_f32(np.asarray(h, dtype=np.uint16)).astype(np.float64)


def ulp_f32(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 23)


def ulp_bf16(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


# ---------------------------------------------------------------- the table
def test_table_hand_values():
    g = kv("rope_table_hand.txt")
    theta, dim = float(g.pop("theta")), int(g.pop("dim"))
    entries = {tuple(int(t) for t in k.split()): [float(v) for v in val.split()]
               for k, val in g.items()}
    n_pos = max(p for p, _ in entries) + 1
    tab = O.rope_table(theta, dim, n_pos)
    assert tab.shape == (n_pos, dim // 2, 2) and tab.dtype == np.float32
    for (p, i), (c, s) in entries.items():
        assert tab[p, i, 0] == np.float32(c), (p, i, tab[p, i, 0], c)
        assert tab[p, i, 1] == np.float32(s), (p, i, tab[p, i, 1], s)


def test_table_position_zero_is_identity():
    tab = O.rope_table(10000.0, 64, 1)
    assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)


def test_table_unit_modulus_and_phase():
    theta, dim = 10000.0, 64
    tab = O.rope_table(theta, dim, 4096).astype(np.float64)
    mod = tab[..., 0] ** 2 + tab[..., 1] ** 2
    assert np.max(np.abs(mod - 1.0)) <= 2.0 ** -22
    # at p = 1 the angle is the frequency itself (all below pi/2 except pair 0)
    freq = np.array([theta ** (-2.0 * i / dim) for i in range(dim // 2)])
    ang = np.arctan2(tab[1, :, 1], tab[1, :, 0])
    assert np.max(np.abs(ang - freq) / freq) <= 2.0 ** -20


def test_table_angle_addition():
    """R_{p+q} = R_p R_q: the product of two entries, in double, matches the
    entry at the summed position to the binary32 roundings involved."""
    tab = O.rope_table(10000.0, 64, 8192).astype(np.float64)
    z = tab[..., 0] + 1j * tab[..., 1]
    rng = np.random.default_rng(7)
    for p, q in rng.integers(0, 4096, size=(64, 2)):
        err = np.abs(z[p] * z[q] - z[p + q])
        assert np.max(err) <= 4 * 2.0 ** -24, (p, q, np.max(err))


def test_table_large_positions_against_libm():
    """Pair 0 turns by exactly one radian per position: cos p and sin p from
    the C library in double, rounded to binary32, agree within one binary32
    ulp at positions up to 2^17."""
    ps = np.array([0, 1, 2, 3, 511, 4095, 32767, 65535, 99991, 131071], dtype=np.int64)
    tab = O.rope_table(10000.0, 64, int(ps.max()) + 1)
    for p in ps:
        c, s = math.cos(float(p)), math.sin(float(p))
        assert abs(float(tab[p, 0, 0]) - c) <= ulp_f32(c) + 2.0 ** -40
        assert abs(float(tab[p, 0, 1]) - s) <= ulp_f32(s) + 2.0 ** -40


def test_table_other_theta_and_dim():
    """The config's compressed layers use theta 160000 (with YaRN, outside the
    ratio-0 table); the ladder itself is pinned at another theta and dim."""
    tab = O.rope_table(160000.0, 16, 3)
    for i in range(8):
        f = 160000.0 ** (-2.0 * i / 16)
        assert tab[1, i, 0] == np.float32(math.cos(f)) or \
            abs(tab[1, i, 0] - math.cos(f)) <= ulp_f32(math.cos(f))
        assert abs(tab[2, i, 1] - math.sin(2 * f)) <= ulp_f32(math.sin(2 * f))


def test_table_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.rope_table(10000.0, 63, 4)
    with pytest.raises(ValueError):
        O.rope_table(0.0, 64, 4)


# ---------------------------------------------------------------- rotation
def rotate_cases():
    it = iter(lines("rope_rotate_hand.txt"))
    for ln in it:
        assert ln.startswith("in:")
        x = [num(t) for t in ln[3:].split()]
        tab = [num(t) for t in next(it).split(":", 1)[1].split()]
        inv = int(next(it).split(":", 1)[1])
        out = [num(t) for t in next(it).split(":", 1)[1].split()]
        yield x, tab, inv, out


def test_rotation_hand_values():
    n = 0
    for x, tab, inv, out in rotate_cases():
        rope_dim = len(tab)
        table = np.array(tab, dtype=np.float32).reshape(1, rope_dim // 2, 2)
        got = O.rope_rows(bf16([x]), table, [0], rope_dim, inverse=bool(inv))
        assert np.array_equal(got, bf16([out])), (x, tab, inv, f64(got))
        n += 1
    assert n == 4


def unit_table(seed, n_pos, half):
    return synth.unit_pairs_f32(seed, synth.TAG_MISC, (n_pos, half))


def test_rotation_matches_exact_complex_product():
    """Within half a bf16 ulp of the exact rotation plus the binary32 error
    of two products and a sum."""
    rng_rows, D, rd = 300, 96, 32
    x = synth.normal_bf16(11, synth.TAG_Q, (rng_rows, D))
    tab = unit_table(12, 50, rd // 2)
    pos = np.arange(rng_rows) % 50
    for inverse in (False, True):
        got = f64(O.rope_rows(x, tab, pos, rd, inverse=inverse))
        xs = f64(x)
        z = xs[:, D - rd::2] + 1j * xs[:, D - rd + 1::2]
        t = tab[pos].astype(np.float64)
        r = t[..., 0] + 1j * (-t[..., 1] if inverse else t[..., 1])
        e = z * r
        exact = np.empty((rng_rows, rd))
        exact[:, 0::2], exact[:, 1::2] = e.real, e.imag
        mag = np.repeat(np.abs(z), 2, axis=1)
        bound = 0.5 * ulp_bf16(exact) + 2.0 ** -22 * mag
        assert np.all(np.abs(got[:, D - rd:] - exact) <= bound)
        assert np.array_equal(got[:, :D - rd], xs[:, :D - rd])


def test_rotation_identity_at_position_zero():
    x = synth.normal_bf16(13, synth.TAG_Q, (64, 512))
    x[x & 0x7FFF == 0] = 0x3F80  # no zeros: -0 minus -0 would give +0
    tab = O.rope_table(10000.0, 64, 2)
    assert np.array_equal(O.rope_rows(x, tab, np.zeros(64, np.int64), 64), x)


def test_rotation_pairs_are_adjacent_values():
    """A table that turns only pair j by 90 degrees changes exactly the values
    2j and 2j+1 of the rotated part (not j and j + rope_dim/2)."""
    D, rd = 64, 16
    x = synth.normal_bf16(14, synth.TAG_Q, (1, D))
    for j in range(rd // 2):
        tab = np.zeros((1, rd // 2, 2), np.float32)
        tab[0, :, 0] = 1.0
        tab[0, j] = (0.0, 1.0)
        got = O.rope_rows(x, tab, [0], rd)
        changed = np.nonzero(got[0] != x[0])[0]
        s = D - rd + 2 * j
        assert set(changed) <= {s, s + 1}
        assert got[0, s] == x[0, s + 1] ^ 0x8000 and got[0, s + 1] == x[0, s]


def test_inverse_undoes_forward():
    x = synth.normal_bf16(15, synth.TAG_Q, (200, 512))
    tab = O.rope_table(10000.0, 64, 4096)
    pos = synth.stream_u64(16, synth.TAG_MISC, 200) % np.uint64(4096)
    y = O.rope_rows(O.rope_rows(x, tab, pos, 64), tab, pos, 64, inverse=True)
    xs, ys = f64(x), f64(y)
    pair = np.repeat(np.hypot(xs[:, 448::2], xs[:, 449::2]), 2, axis=1)
    assert np.all(np.abs(ys[:, 448:] - xs[:, 448:]) <= 2.0 ** -7 * pair)
    assert np.array_equal(y[:, :448], x[:, :448])


def test_rotation_preserves_pair_norm():
    x = synth.normal_bf16(17, synth.TAG_Q, (100, 128))
    tab = O.rope_table(10000.0, 64, 100)
    got = f64(O.rope_rows(x, tab, np.arange(100), 64))
    xs = f64(x)
    n0 = np.hypot(xs[:, 64::2], xs[:, 65::2])
    n1 = np.hypot(got[:, 64::2], got[:, 65::2])
    assert np.all(np.abs(n1 - n0) <= 2.0 ** -7 * n0 + 1e-30)


def test_rope_fp8_is_rotation_then_fp8():
    x = synth.normal_bf16(18, synth.TAG_KV_NEW, (40, 512))
    tab = O.rope_table(10000.0, 64, 40)
    pos = np.arange(40)
    got = O.rope_fp8_rows(x, tab, pos, 64)
    assert np.array_equal(got, O.fp8_round_rows(O.rope_rows(x, tab, pos, 64)))
    # at position 0 the rotation is the identity and only the fp8 step is left
    x0 = x.copy()
    x0[x0 & 0x7FFF == 0] = 0x3F80
    assert np.array_equal(O.rope_fp8_rows(x0, tab, np.zeros(40, np.int64), 64),
                          O.fp8_round_rows(x0))


def test_rotation_rejects_bad_arguments():
    x = synth.normal_bf16(19, synth.TAG_Q, (2, 64))
    tab = O.rope_table(10000.0, 16, 4)
    with pytest.raises(ValueError):
        O.rope_rows(x, tab, [0, 4], 16)          # position outside the table
    with pytest.raises(ValueError):
        O.rope_rows(x, tab, [0], 16)             # one position per row
    with pytest.raises(ValueError):
        O.rope_rows(x, tab, [0, 1], 32)          # table width != rope_dim / 2
