"""Pins for the oracle's element and scale codecs (CPU only)."""

from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O
from conftest import read_golden
from fp_exact import e4m3_grid, nearest


def _golden_map():
    return {row[0]: row[1:] for row in read_golden("formats.txt")}


def _e2m1_signed_grid():
    mags = [F(v) for v in _golden_map()["E2M1"]]
    grid = [(m, i) for i, m in enumerate(mags)]
    grid += [(-m, 8 | i) for i, m in enumerate(mags) if i]
    return grid


def test_e2m1_values_match_table6():
    mags = [float(v) for v in _golden_map()["E2M1"]]
    assert O.e2m1_value(np.arange(8)).tolist() == mags
    assert O.e2m1_value(np.arange(8, 16)).tolist() == [-m for m in mags]


def test_e2m1_codes_match_table7():
    for row in read_golden("table7_group.txt"):
        q, code = float(row[1]), int(row[2], 2)
        assert O.e2m1_value(code) == q
        assert O.e2m1_encode(np.float32(q)) == code


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16)
    back = O.e2m1_encode(O.e2m1_value(codes))
    expect = np.where(codes == 8, 0, codes)        # -0 comes back as canonical +0
    assert back.tolist() == expect.tolist()


def test_e2m1_midpoints_ties_to_even():
    mids = [float(v) for v in read_golden("adamx_midpoints.txt")[0]]
    got = O.e2m1_value(O.e2m1_encode(np.array(mids, np.float32)))
    # each midpoint lies between two magnitudes, one with an even mantissa bit
    assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    got_neg = O.e2m1_value(O.e2m1_encode(-np.array(mids, np.float32)))
    assert got_neg.tolist() == [0.0, -1.0, -1.0, -2.0, -2.0, -4.0, -4.0]
    up = np.nextafter(np.array(mids, np.float32), np.float32(10))
    assert O.e2m1_value(O.e2m1_encode(up)).tolist() == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_bruteforce_random():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.normal(0, 2.5, 3000).astype(np.float32),
        (rng.integers(-28, 29, 400) / 4.0).astype(np.float32),   # grid points and midpoints
        np.array([6.0, 6.5, 7.9, 100.0, -100.0, 0.0, -0.0], np.float32),
    ])
    grid = _e2m1_signed_grid()
    codes = O.e2m1_encode(vals)
    for v, c in zip(vals, codes):
        _, want = nearest(F(float(v)), grid, lambda code: (code & 1) == 0)
        if want == 8:
            want = 0
        assert int(c) == want, (float(v), int(c), want)


def test_e4m3_range_and_roundtrip():
    lo, hi = (float(v) for v in _golden_map()["E4M3_RANGE"])
    vals = O.e4m3_value(np.arange(0x7F))
    assert vals[1] == lo and vals[-1] == hi
    assert np.all(np.diff(vals) > 0)
    assert O.e4m3_encode(vals).tolist() == list(range(0x7F))
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))
    grid = dict((code, val) for val, code in e4m3_grid())
    assert all(F(float(O.e4m3_value(c))) == grid[c] for c in range(0x7F))


def test_e4m3_bruteforce_random():
    rng = np.random.default_rng(12)
    b = np.concatenate([
        np.exp2(rng.uniform(-12, 9.2, 3000)).astype(np.float32),
        np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 448.0, 460.0, 464.0, 1e6], np.float32),
    ])
    grid = e4m3_grid()
    # exact midpoints between neighbouring grid values
    g = sorted(v for v, _ in grid)
    mids = [float((g[i] + g[i + 1]) / 2) for i in range(0, len(g) - 1, 7)]
    b = np.concatenate([b, np.array(mids, np.float32)])
    codes = O.e4m3_encode(b)
    for x, c in zip(b, codes):
        _, want = nearest(min(F(float(x)), F(448)), grid, lambda code: (code & 1) == 0)
        assert int(c) == want, (float(x), int(c), want)


def test_offset_select_bruteforce():
    rng = np.random.default_rng(13)
    r = np.concatenate([rng.uniform(-1.5, 1.5, 2000),
                        np.array([1 / 16, -1 / 16, -3 / 16, 3 / 16, 0.0, 5 / 16, -5 / 16, 1.0, -1.0])])
    d = O.offset_select(r)
    for x, got in zip(r, d):
        best = None
        for cand in (0, 1, -1, -2):                   # smaller |d| first on ties
            dist = abs(F(float(x)) - F(cand, 8))
            if best is None or dist < best[0]:
                best = (dist, cand)
        assert int(got) == best[1]
    # the boundaries of the decision fall exactly midway between neighbouring deltas
    assert O.offset_select(np.array([1 / 16, -1 / 16, -3 / 16])).tolist() == [0, 0, -1]


def test_offset_codes_and_deltas():
    gm = _golden_map()
    codes = dict(item.split(":") for item in gm["OFFSETS"])
    for d_str, bits in codes.items():
        byte = O.pack_offsets_byte(np.array([int(d_str)] * 4))
        assert (int(byte) & 3) == int(bits, 2)
    assert sorted(F(d, 8) for d in (-2, -1, 0, 1)) == sorted(F(x) for x in gm["DELTA"])


def test_autofp2_digits():
    gm = _golden_map()
    mags = [float(v) for v in gm["E2M1"]]
    digits = O.autofp2_digit(np.arange(8))
    absorbed = sorted(m for m, q in zip(mags, digits) if q == 1)
    assert absorbed == [float(v) for v in gm["AUTOFP2_DIGIT1"]]
    levels = sorted(set((2 * O.autofp2_digit(np.arange(16))).tolist()))
    assert levels == [int(v) for v in gm["AUTOFP2_LEVELS"]]
    # sign kept: code with sign bit set gives the negated digit (and -0 -> 0)
    assert (O.autofp2_digit(np.arange(8, 16)) == -digits).all()


@pytest.mark.parametrize("bad", [-1.0, float("nan")])
def test_e4m3_rejects_negative(bad):
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([bad]))
