"""Pins of the oracle's fp8 round trip (CPU only).

What fixes the expected values: the act_quant_inplace and pow2_ceil contracts
and the precision paragraph of the "deepseek_v41_ref::attn" rustdoc (result
bf16-exact e4m3 x 2^k, block 32, power-of-two scale from amax/448 with amax
floored at 1e-4, round to nearest even, clamping), and the OCP E4M3FN format.
The checks below re-derive the grid by enumerating the 256 e4m3 codes (the
oracle uses a quantum formula instead), hand-derived block values, and the
exhaustive set of finite bf16 inputs.
"""
import math

import numpy as np
import pytest

import oracle as O
from golden_io import exact_bf16, kv, lines, num

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def e4m3fn_table():
    """All finite E4M3FN values from the OCP bit layout: s eeee mmm, bias 7,
    e = 0 subnormal (m/8 * 2^-6), e = 15 with m = 7 is NaN (no infinities)."""
    vals, codes = [], []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-mag if s else mag)
        codes.append(code)
    return np.array(vals), np.array(codes)


def nearest_e4m3_even(y):
    """Nearest table value to y (|y| <= 448); halfway -> the even code."""
    vals, codes = e4m3fn_table()
    pos = vals >= 0
    pv, pc = vals[pos], codes[pos]
    order = np.argsort(pv, kind="stable")
    pv, pc = pv[order], pc[order]
    a = np.abs(y)
    hi = np.clip(np.searchsorted(pv, a, side="left"), 0, len(pv) - 1)
    lo = np.clip(hi - 1, 0, len(pv) - 1)
    dlo, dhi = a - pv[lo], pv[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pc[hi] % 2 == 0))
    r = np.where(pick_hi, pv[hi], pv[lo])
    r = np.where(a == pv[hi], pv[hi], r)
    return np.copysign(r, y)


def bf16_to_f64(h):
    h = np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return h.view(np.float32).astype(np.float64)


def expected_block(xb):
    """Re-derivation of one block's expected output by table lookup."""
    amax = np.float32(np.max(np.abs(xb))) if xb.size else np.float32(0)
    amax = max(amax, np.float32(1e-4))
    ratio = np.float32(amax) / np.float32(448.0)       # binary32 division
    m, e = math.frexp(float(ratio))
    scale = math.ldexp(1.0, e - 1) if m == 0.5 else math.ldexp(1.0, e)
    y = np.clip(xb / scale, -448.0, 448.0)
    out = nearest_e4m3_even(y) * scale
    # e * 2^k is on the bf16 grid unless it reaches 2^128 (a block whose amax
    # lies within the last e4m3 step of the bf16 maximum): then the final
    # rounding to bf16 overflows to +-inf.
    out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, out), out)
    return out, scale


def test_e4m3_table_shape():
    vals, _ = e4m3fn_table()
    assert len(vals) == 254
    assert vals.max() == 448.0 and vals.min() == -448.0
    assert np.min(np.abs(vals[vals != 0])) == 2.0 ** -9


def test_e4m3_round_matches_enumeration():
    # every bf16 value in [-448, 448] plus every midpoint of the grid
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f64(allb)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    vals, _ = e4m3fn_table()
    pv = np.unique(np.abs(vals))
    mids = (pv[1:] + pv[:-1]) / 2
    ys = np.concatenate([x, mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    got = np.array([O.e4m3_round(float(v)) for v in ys])
    want = nearest_e4m3_even(ys)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_pow2_ceil_values():
    assert O.pow2_ceil(1.0) == 1.0
    assert O.pow2_ceil(np.nextafter(np.float32(1.0), np.float32(2.0))) == 2.0
    assert O.pow2_ceil(0.75) == 1.0
    assert O.pow2_ceil(2.0 ** -22) == 2.0 ** -22
    assert O.pow2_ceil(1.5 * 2.0 ** -22) == 2.0 ** -21
    rng = np.random.default_rng(1)
    v = (rng.uniform(0.5, 2.0, 2000) * 2.0 ** rng.integers(-100, 100, 2000)).astype(np.float32)
    for x in v:
        m, e = math.frexp(float(x))
        want = math.ldexp(1.0, e - 1) if m == 0.5 else math.ldexp(1.0, e)
        assert O.pow2_ceil(float(x)) == want


def read_cases():
    ls = list(lines("fp8_closed_form.txt"))
    assert len(ls) % 2 == 0
    for a, b in zip(ls[0::2], ls[1::2]):
        assert a.startswith("in:") and b.startswith("out:")
        xin = [num(t) for t in a[3:].split()]
        xout = [num(t) for t in b[4:].split()]
        yield xin, xout


def test_closed_form_blocks():
    n = 0
    for xin, xout in read_cases():
        blk = np.zeros(32, dtype=np.uint16)
        want = np.zeros(32, dtype=np.uint16)
        for i, v in enumerate(xin):
            blk[i] = exact_bf16(v)
        for i, v in enumerate(xout):
            want[i] = exact_bf16(v)
        got = O.fp8_round_rows(blk[None, :])[0]
        assert np.array_equal(got, want), (xin, got, want)
        n += 1
    assert n >= 6


def test_exhaustive_bf16_property():
    """Every finite bf16 input, in blocks of 32 (sorted, so the scales span the
    whole range, and shuffled): the output is bf16-exact e * 2^k with e an
    E4M3FN value, |e| <= 448, k shared by the block, e the nearest to x / 2^k
    with ties to the even code, and the sign of x kept (zeros included)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f64(allb)
    fin = allb[np.isfinite(x)]
    n = (fin.size // 32) * 32
    sorted_rows = fin[np.argsort(bf16_to_f64(fin), kind="stable")][:n].reshape(-1, 32)
    rng = np.random.default_rng(7)
    shuffled = rng.permutation(fin)[:n].reshape(-1, 32)
    rows = np.concatenate([sorted_rows, shuffled])
    # one row per block keeps the cases independent; also a wide row of 16 blocks
    got = O.fp8_round_rows(rows)
    wide = O.fp8_round_rows(rows[:64].reshape(4, 512))
    assert np.array_equal(wide.reshape(-1, 32), got[:64])
    vals, _ = e4m3fn_table()
    vset = set(vals.tolist())
    xin = bf16_to_f64(rows)
    xout = bf16_to_f64(got)
    n_overflow = 0
    for r in range(rows.shape[0]):
        want, scale = expected_block(xin[r])
        assert np.array_equal(xout[r], want), r
        assert np.array_equal(np.signbit(xout[r]), np.signbit(xin[r])), r
        fin = np.isfinite(xout[r])
        e = xout[r][fin] / scale
        assert all(v in vset for v in e.tolist())
        assert np.max(np.abs(e), initial=0.0) <= 448.0
        n_overflow += int((~fin).sum())
    # only the blocks at the very top of the bf16 range overflow
    assert 0 < n_overflow < 64


def test_row_len_must_be_block_multiple():
    with pytest.raises(ValueError):
        O.fp8_round_rows(np.zeros((1, 48), dtype=np.uint16))


def test_in_place_idempotent():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((8, 512)) * 3).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    once = O.fp8_round_rows(b)
    twice = O.fp8_round_rows(once)
    assert np.array_equal(once, twice)
