"""Pins of the refinement-aware GPTQ oracle (oracle/gptq_ref.py, [AE] App. E,
Algorithm 1 and Eq. 7), CPU only. What fixes them, independently of the
oracle's code:
  - the identity Hessian: no propagation (U = I) and equal column weights
    reduce Algorithm 1 to the AutoFP6 weight encoder with the budgeted mask,
    which tests/test_oracle_*.py pin on their own;
  - the closed form of optimal compensation: quantizing the columns J of the
    remaining block and minimising the Hessian-weighted error over the later
    columns moves them by -(W_J - Q_J) [Hinv]_JJ^-1 [Hinv]_J,later, with Hinv
    the explicit inverse of the trailing Hessian block (np.linalg.inv);
  - brute force with exact rationals: the mask of line 20 minimises Eq. 7
    over every mask of its size; the greedy allocation of lines 5-12 attains
    the least total error over every allocation of the budget;
  - the factor's definition U^T U = H_d^-1, U upper triangular;
  - the purpose of the pass: a lower Hessian-weighted output error than
    rounding each weight alone, on correlated calibration inputs.
"""

import itertools
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle as O
from oracle import gptq_ref as P
from runtime_mixed_precision_amd import synthetic as S


def weights(n, k, seed):
    return S.weights(n, k, seed=seed, tensor_id=1).numpy()


def damped_hessian(k, tokens=512, seed=0):
    x = S.calibration(tokens, k, seed=seed, tensor_id=2).numpy()
    return P.dampen(P.hessian(x))


def test_factor_is_the_cholesky_factor_of_the_inverse():
    hd = damped_hessian(64)
    u = P.inverse_factor(hd)
    assert np.all(np.tril(u, -1) == 0) and np.all(np.diag(u) > 0)
    assert np.abs(u.T @ u @ hd - np.eye(64)).max() < 1e-9


@pytest.mark.parametrize("n,k,seed", [(32, 128, 0), (64, 256, 1), (16, 1024, 2), (7, 48, 3)])
def test_identity_hessian_is_the_autofp6_encoder(n, k, seed):
    w = weights(n, k, seed)
    out = P.gptq_quantize(w, np.eye(k), np.ones(k))
    bits, r = O.select_weight_mask(w, 0.2)
    ref = O.quantize_weight(w, O.pack_nibbles(bits))
    for key in ("codes", "scales", "mask", "offsets"):
        assert np.array_equal(out[key], ref[key]), key
    assert out["T"] == ref["T"] and out["n_refined"] == r
    assert np.array_equal(out["What"], O.decode_weight(ref, 6))


@pytest.mark.parametrize("j", [0, 1, 2])
def test_update_is_the_optimal_compensation(j):
    n, k = 5, 64
    rng = np.random.default_rng(j)
    w = rng.standard_normal((n, k))
    hd = damped_hessian(k, seed=4)
    u = P.inverse_factor(hd)
    J = slice(16 * j, 16 * (j + 1))
    q = np.round(w[:, J], 1)
    e = P.solve_group_error(w[:, J] - q, u[J, J])
    w2 = P.propagate(w, e, u, j)
    hinv = np.linalg.inv(hd[16 * j:, 16 * j:])
    delta = -(w[:, J] - q) @ np.linalg.inv(hinv[:16, :16]) @ hinv[:16, 16:]
    assert np.array_equal(w2[:, :16 * (j + 1)], w[:, :16 * (j + 1)])
    assert np.allclose(w2[:, 16 * (j + 1):], w[:, 16 * (j + 1):] + delta, rtol=1e-9, atol=1e-9)


def exact_error(w_j, what, h_j):
    return sum(F(float(h_j[i])) * sum((F(float(w_j[r, i])) - F(float(what[r, i]))) ** 2
                                      for r in range(w_j.shape[0])) for i in range(16))


def exact_masked(mask, w4, wr):
    sel = np.repeat([(mask >> s) & 1 for s in range(4)], 4).astype(bool)
    return np.where(sel[None, :], wr, w4)


@pytest.mark.parametrize("seed", range(6))
def test_line20_mask_minimises_eq7(seed):
    rng = np.random.default_rng(100 + seed)
    w = (rng.standard_normal((3, 16)) * 0.05).astype(np.float32).astype(np.float64)
    h = rng.uniform(0.1, 3.0, 16)
    _, _, _, w4, wr = P.encode_group(w, np.abs(w).max())
    for level in (1, 2):
        m = P.best_mask(w, w4, wr, h, level)
        errs = {sum(1 << s for s in c): exact_error(w, exact_masked(sum(1 << s for s in c), w4, wr), h)
                for c in itertools.combinations(range(4), level)}
        best = min(errs.values())
        assert errs[m] == best
        first = next(mm for mm in sorted(errs, key=lambda mm: [s for s in range(4) if (mm >> s) & 1])
                     if errs[mm] == best)
        assert m == first


@pytest.mark.parametrize("rho,seed", [(0.2, 0), (0.4, 1), (0.5, 2), (0.1, 3)])
def test_allocation_attains_the_least_total_error(rho, seed):
    n, k = 6, 64
    w = weights(n, k, 10 + seed)
    h = np.diag(damped_hessian(k, seed=seed))
    levels, _ = P.allocate_levels(w, h, rho)
    budget = min(int(np.floor(rho * k / 4)), 2 * (k // 16))
    assert levels.sum() == budget and levels.max() <= 2
    w64 = w.astype(np.float64)
    amax = np.abs(w).max()
    L = []
    for j in range(k // 16):
        J = slice(16 * j, 16 * (j + 1))
        _, _, _, w4, wr = P.encode_group(w64[:, J], amax)
        L.append([min(exact_error(w64[:, J], exact_masked(sum(1 << s for s in c), w4, wr), h[J])
                      for c in itertools.combinations(range(4), lv)) for lv in range(3)])
    best = min(sum(L[j][a[j]] for j in range(len(L)))
               for a in itertools.product(range(3), repeat=len(L)) if sum(a) == budget)
    assert sum(L[j][levels[j]] for j in range(len(L))) == best


def test_mask_matches_levels_and_budget():
    n, k = 24, 256
    w = weights(n, k, 5)
    hd = damped_hessian(k, seed=5)
    out = P.gptq_quantize(w, P.inverse_factor(hd), np.diag(hd))
    pop = np.array([bin(int(b)).count("1") for b in out["mask_bits"]])
    assert np.array_equal(pop, out["levels"])
    assert out["n_refined"] == int(np.floor(0.2 * k / 4)) == out["offsets"].shape[1]


def test_gptq_lowers_the_hessian_weighted_error():
    """Correlated calibration inputs: the compensated pass leaves a much lower
    tr((W - What) H_d (W - What)^T) than encoding each weight alone with the
    same mask (measured: 17 % lower), and U = I reproduces the latter exactly."""
    n, k = 32, 256
    w = weights(n, k, 6)
    hd = damped_hessian(k, tokens=1024, seed=6)
    out = P.gptq_quantize(w, P.inverse_factor(hd), np.diag(hd))
    rtn = O.decode_weight(O.quantize_weight(w, out["mask"]), 6)
    e_gptq = P.hessian_weighted_error(w, out["What"], hd)
    e_rtn = P.hessian_weighted_error(w, rtn, hd)
    assert e_gptq < 0.9 * e_rtn, (e_gptq, e_rtn)
    plain = P.gptq_quantize(w, np.eye(k), np.diag(hd))
    assert np.array_equal(plain["What"], O.decode_weight(O.quantize_weight(w, plain["mask"]), 6))
