"""Pins of the oracle's NVFP4 / AutoFP6 encoders and the weight mask (CPU only).

NVFP4 at the 4-bit level is textbook NVFP4 ([AE] App. B.1, Eqs. 2-3); these
tests recompute it with exact rationals and an independent binary32 rounding.
"""

import itertools
import math
from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O
from conftest import read_golden
from fp_exact import e4m3_grid, nearest, round_f32


def _e2m1_grid():
    mags = [F(v) for v in {r[0]: r[1:] for r in read_golden("formats.txt")}["E2M1"]]
    return [(m, i) for i, m in enumerate(mags)] + [(-m, 8 | i) for i, m in enumerate(mags) if i]


def _even(code):
    return (code & 1) == 0


def brute_nvfp4(x):
    """Eqs. 2-3 with exact rationals and each fp32 step rounded by round_f32."""
    rows, K = x.shape
    xs = [[F(float(v)) for v in row] for row in x]
    amax = max((abs(v) for row in xs for v in row), default=F(0))
    T = round_f32(amax / 2688)
    six_t = round_f32(6 * T)
    g2 = _e2m1_grid()
    g4 = e4m3_grid()
    codes = np.zeros((rows, K), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    for r in range(rows):
        for j in range(K // 16):
            grp = xs[r][16 * j:16 * j + 16]
            a = max(abs(v) for v in grp)
            b = round_f32(a / six_t) if six_t else F(0)
            Bv, Bc = nearest(min(b, F(448)), g4, _even)
            scales[r, j] = Bc
            s = round_f32(T * Bv)
            for i, v in enumerate(grp):
                vv = round_f32(v / s) if s else F(0)
                _, c = nearest(vv, g2, _even)
                codes[r, 16 * j + i] = 0 if c == 8 else c
    return codes, scales, T


@pytest.mark.parametrize("case", ["normal", "outliers", "midpoints", "tiny_groups", "mixed_scale"])
def test_nvfp4_matches_exact_bruteforce(case):
    rng = np.random.default_rng(abs(hash(case)) % 1000)
    if case == "normal":
        x = rng.standard_normal((3, 32))
    elif case == "outliers":
        x = rng.standard_normal((3, 48))
        x.flat[rng.choice(x.size, 3, replace=False)] *= 20
    elif case == "midpoints":
        # s = 0.25 exactly (see Table 7): x/s lands on E2M1 midpoints and grid points
        x = 0.25 * (rng.integers(-24, 25, (2, 32)) / 4.0)
        x[:, 0] = 1.5
        x[:, 16] = -1.5
    elif case == "tiny_groups":
        x = rng.standard_normal((2, 64))
        x[0, 16:32] *= 1e-5            # group scale underflows to zero
        x[1, 32:48] = 0.0              # all-zero group
    else:
        x = rng.standard_normal((2, 64)) * np.exp2(rng.integers(-6, 7, (2, 64)))
    x = x.astype(np.float32)
    base = O.nvfp4_quantize(x)
    codes, scales, T = brute_nvfp4(x)
    assert F(float(base.T)) == T
    assert (base.scales == scales).all()
    assert (base.codes == codes).all()


def test_zero_tensor_and_zero_groups():
    base = O.nvfp4_quantize(np.zeros((2, 32), np.float32))
    assert float(base.T) == 0.0 and not base.codes.any() and not base.scales.any()
    x = np.ones((1, 48), np.float32)
    x[0, 16:32] = 0
    x[0, 32:48] = 1e-6                 # b = 1e-6 * 448 < 2^-10 -> B = 0
    base = O.nvfp4_quantize(x)
    assert base.scales[0].tolist() == [0x7E, 0, 0]
    assert not base.codes[0, 16:].any()


def test_saturation_when_scale_rounds_down():
    # amax_j / (6T) = 448 * 0.96 rounds down to E4M3 416 -> x/(TB) > 6 -> code 6
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16] = 0.96
    base = O.nvfp4_quantize(x)
    assert O.e4m3_value(base.scales[0, 1]) == 416.0
    assert float(base.v[0, 16]) > 6.0
    assert int(base.codes[0, 16]) == 0b0111


def test_quantization_error_bounds():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    base = O.nvfp4_quantize(x)
    q = O.e2m1_value(base.codes)
    v = base.v.astype(np.float64)
    gap = {0.0: 0.25, 0.5: 0.25, 1.0: 0.25, 1.5: 0.25, 2.0: 0.5, 3.0: 0.5, 4.0: 1.0, 6.0: np.inf}
    half = np.vectorize(lambda a: gap[a])(np.abs(q))
    inside = np.abs(v) <= 6
    assert (np.abs(v - q)[inside] <= half[inside]).all()
    d = O.offset_select(v - q)
    assert (np.abs(v - q - d / 8.0) <= np.abs(v - q)).all()     # never moves farther
    # Below 2 the fixed step 1/8 is the E2M3 step (§3.2): where the residual is
    # within the offsets' reach, q + d/8 is an E2M3 value nearest to v.
    e2m3 = np.array([float(t) for t in {r[0]: r[1:] for r in read_golden("formats.txt")}["E2M3"]])
    e2m3 = np.concatenate([-e2m3[::-1], e2m3])
    r = v - q
    sel = (np.abs(v) < 1.875) & (r >= -0.25) & (r < 3 / 16)
    assert sel.sum() > 1000
    best = np.min(np.abs(v[sel][:, None] - e2m3[None, :]), axis=1)
    assert (np.abs(v[sel] - (q + d / 8.0)[sel]) == best).all()
    assert np.isin((q + d / 8.0)[sel], e2m3).all()


def test_activation_mask_respects_weight_mask():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    base = O.nvfp4_quantize(x)
    ex = rng.integers(0, 16, 128 // 16)
    ex = np.array([b if bin(b).count("1") <= 2 else b & 0b0011 for b in ex])
    bits, d = O.activation_refinement(base, ex, 0.003)
    assert not (bits & ex[None, :]).any()
    free_bits, _ = O.activation_refinement(base, None, 0.003)
    assert ((free_bits & ~ex[None, :]) == bits).all()
    # a lower threshold refines a superset
    lo_bits, _ = O.activation_refinement(base, None, 0.0005)
    assert ((lo_bits & free_bits) == free_bits).all()


def _exact_group_error(w, base, j, mask_bits):
    """E_j(m) of Alg. 1 with H = I, exact: sum over rows of squared error of
    group j, dequantized as T B q, or T B (q + delta) on the subgroups of m."""
    tot = F(0)
    T = F(float(base.T))
    for n in range(w.shape[0]):
        B = F(float(O.e4m3_value(base.scales[n, j])))
        for i in range(16):
            k = 16 * j + i
            q = F(float(O.e2m1_value(base.codes[n, k])))
            if (mask_bits >> (i // 4)) & 1:
                r = F(float(base.v[n, k])) - q
                best = min((abs(r - F(c, 8)), c) for c in (0, 1, -1, -2))
                q = q + F(best[1], 8)
            tot += (F(float(w[n, k])) - T * B * q) ** 2
    return tot


@pytest.mark.parametrize("seed,K,budget", [(0, 32, 1), (1, 32, 2), (2, 32, 3), (3, 48, 4), (4, 48, 2)])
def test_weight_mask_matches_exact_algorithm(seed, K, budget):
    """Alg. 1 allocation (greedy over L_j(l) = min_{|m| = l} E_j(m)) evaluated
    exactly, then each group's mask m* = argmin over masks with l_j bits."""
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((3, K))).astype(np.float32)
    base = O.nvfp4_quantize(w)
    G = K // 16
    masks_by_l = {l: [m for m in range(16) if bin(m).count("1") == l] for l in (0, 1, 2)}
    E = {(j, m): _exact_group_error(w, base, j, m) for j in range(G) for m in range(16)}
    L = {(j, l): min(E[(j, m)] for m in masks_by_l[l]) for j in range(G) for l in (0, 1, 2)}
    level = [0] * G
    for _ in range(budget):
        cands = [(L[(j, level[j])] - L[(j, level[j] + 1)], -j) for j in range(G) if level[j] < 2]
        _, mj = max(cands)
        level[-mj] += 1
    want = [min(masks_by_l[level[j]], key=lambda m: (E[(j, m)], m)) for j in range(G)]
    # also the global optimum under the per-group cap
    best = min((sum(L[(j, a[j])] for j in range(G)), a)
               for a in itertools.product((0, 1, 2), repeat=G) if sum(a) == budget)
    assert sum(L[(j, level[j])] for j in range(G)) == best[0]

    g = O.weight_subgroup_gains(w, base)
    col = g.sum(axis=0)
    got = O.greedy_weight_mask(col.reshape(G, 4), budget)
    assert got.tolist() == want
    rho = budget * 4 / K
    bits, R = O.select_weight_mask(w, rho + 1e-9)
    assert R == budget and bits.tolist() == want


def test_weight_mask_closed_form_topr():
    """Greedy over non-increasing marginal gains = top-R of (group, rank) with
    at most two per group, ordered by gain, then group, then subgroup."""
    rng = np.random.default_rng(9)
    w = (0.02 * rng.standard_normal((64, 1024))).astype(np.float32)
    w[:, rng.choice(1024, 10, replace=False)] *= 3
    base = O.nvfp4_quantize(w)
    col = np.zeros(1024 // 4)
    for row in O.weight_subgroup_gains(w, base):
        col = col + row
    col = col.reshape(-1, 4)
    R = math.floor(0.2 * 1024 / 4)
    got = O.greedy_weight_mask(col, R)
    cands = []
    for j in range(col.shape[0]):
        top2 = sorted(range(4), key=lambda k: (-col[j, k], k))[:2]
        cands += [(-col[j, k], j, k) for k in top2]
    chosen = sorted(cands)[:R]
    want = np.zeros(col.shape[0], np.uint8)
    for _, j, k in chosen:
        want[j] |= 1 << k
    assert (got == want).all()
    assert sum(bin(int(b)).count("1") for b in got) == R
    assert all(bin(int(b)).count("1") <= 2 for b in got)


def test_weight_offsets_compacted_layout():
    rng = np.random.default_rng(6)
    w = (0.02 * rng.standard_normal((5, 96))).astype(np.float32)
    bits, R = O.select_weight_mask(w, 0.2)
    pk = O.quantize_weight(w, O.pack_nibbles(bits))
    assert pk["offsets"].shape == (5, R) and pk["n_refined"] == R
    base = O.nvfp4_quantize(w)
    d = O.offset_select(base.v.astype(np.float64) - O.e2m1_value(base.codes))
    col = 0
    for j in range(96 // 16):
        for k in range(4):
            if (int(bits[j]) >> k) & 1:
                for n in range(5):
                    byte = int(pk["offsets"][n, col])
                    got = [((byte >> (2 * e)) & 3) for e in range(4)]
                    want = [int(v) & 3 for v in d[n, 16 * j + 4 * k:16 * j + 4 * k + 4]]
                    assert got == want
                col += 1
    assert col == R
    tb = float(base.T) * np.repeat(O.e4m3_value(base.scales), 16, axis=1)
    dense = np.zeros_like(d, dtype=np.float64)
    for j in range(6):
        for k in range(4):
            if (int(bits[j]) >> k) & 1:
                dense[:, 16 * j + 4 * k:16 * j + 4 * k + 4] = d[:, 16 * j + 4 * k:16 * j + 4 * k + 4]
    assert (O.decode_weight(pk, 6) == tb * (O.e2m1_value(base.codes) + dense / 8.0)).all()
