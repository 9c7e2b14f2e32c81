"""Exact-arithmetic helpers for pinning the oracle (tests only).

Everything here works on ``fractions.Fraction`` and is written independently of
``oracle/``: an IEEE binary32 round-to-nearest-even of an exact rational, and
brute-force nearest-value searches over explicitly listed grids.
"""

from fractions import Fraction as F


def round_f32(x):
    """Round an exact rational to the nearest IEEE binary32 value (ties to
    even), including the subnormal range; overflow is not handled."""
    x = F(x)
    if x == 0:
        return F(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** max(e - 23, -149)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > F(1, 2) or (rem == F(1, 2) and n % 2 == 1):
        n += 1
    return sgn * n * ulp


def nearest(value, grid, even_of):
    """Member of ``grid`` (list of (exact value, code)) nearest to ``value``;
    among equally near members the one whose ``even_of(code)`` is true."""
    best = None
    for g, code in grid:
        dist = abs(F(value) - g)
        if best is None or dist < best[0] or (dist == best[0] and even_of(code) and not even_of(best[2])):
            best = (dist, g, code)
    return best[1], best[2]


def e4m3_grid():
    """Non-negative finite E4M3 values from the 1/4/3 layout with bias 7
    (subnormals m/8 * 2^-6); code 0x7F is NaN and excluded."""
    out = []
    for e in range(16):
        for m in range(8):
            code = (e << 3) | m
            if code == 0x7F:
                continue
            if e == 0:
                val = F(m, 8) * F(1, 64)
            else:
                val = (1 + F(m, 8)) * F(2) ** (e - 7)
            out.append((val, code))
    return out
