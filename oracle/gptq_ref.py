"""Plain CPU reference of the refinement-aware GPTQ calibration of [AE]
App. E ("Refinement-Aware GPTQ Calibration"), Algorithm 1 with the
diagonal-Hessian-weighted group error of Eq. 7.

TEST INFRASTRUCTURE: imported only by the tests, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg. It shares no code with the HIP library.

Paper: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
Exponent-Mantissa Refinement" (arXiv 2611.10165v1), cited as [AE].

What the algorithm computes (App. E, Alg. 1):
  * line 4: the FP32 tensor scale T = amax(W) / (6 * 448), fixed for the pass;
  * lines 5-12, budget allocation on the original weights: for every group j
    (16 columns J) L_j(l) = min over masks m refining l of its four subgroups
    of E_j(m), l in {0, 1, 2}; then floor(rho K / 4) times, one more refined
    subgroup to the group with the largest L_j(l_j) - L_j(l_j + 1) (l_j < 2);
  * Eq. 7: E_j(m) = sum over i in J of H_ii * ||W[:, i] - What[:, i](m)||^2,
    What(m) the dequantized group with the refined values T B (q + delta) on
    the subgroups of m and the NVFP4 values T B q elsewhere;
  * lines 13-24, the GPTQ pass over the groups in order: B, q and delta of the
    group from the error-compensated weights (lines 15-19), the mask
    m*_j = argmin over masks refining l_j subgroups of E_j (line 20), the
    group's dequantized values (line 21), its error
    E = (W[:, J] - What[:, J]) U_JJ^-1 (line 22) propagated to all later
    columns: W[:, later] -= E U[J, later] (line 23).

Readings (the extracted listing lost lines 1-3 and garbled line 21):
  G1  H = X^T X over calibration activations X [tokens, K] (fp64); the
      dampened H_d = H + lam * mean(diag H) * I with lam = 0.01 (GPTQ's
      default; the pages give none); U is the upper Cholesky factor of
      H_d^-1 (H_d^-1 = U^T U), the matrix lines 22-23 use, as in GPTQ.
  G2  Eq. 7 weighs with the diagonal of the same dampened H_d.
  G3  Line 21 stores What(m*_j) as the group's result; W keeps its
      compensated values for line 22 (otherwise E would be zero).
  G4  Precision: the working weights are fp64. Lines 15-17 encode a group
      from its fp64 values rounded to fp32 with the fp32 steps of Eqs. 2-3
      (``autofp_ref.nvfp4_quantize`` with the tensor scale of line 4) and the
      offsets of ``autofp_ref.offset_select``; What is exact in fp64. Line 22
      is forward substitution, e_i = (r_i - sum_{k<i} e_k U_ki) / U_ii with the
      sum subtracted term by term in k order; line 23 subtracts, per element,
      the 16-term sum E_0 U_0c + ... + E_15 U_15c accumulated in index order.
      Every product and sum is a separate IEEE fp64 operation (no fused
      multiply-add).
  G5  Ties: the masks of M_l are tried in lexicographic order of their
      subgroup indices and the first minimal E_j wins (line 20 and line 6);
      line 10 takes the lowest j on a tie.
  G6  The budget is floor(rho * K / 4) (rho*K/4 in fp64), as the encoder's.

Parity status: pinned by ``tests/test_oracle_gptq.py`` (identity Hessian
reduces to the pinned AutoFP6 encoder; the update against the closed form
of optimal compensation from an explicit inverse; brute force over masks and
allocations with exact rationals; the factor against its definition; the
calibration objective).
"""

from __future__ import annotations

import itertools
import math

import numpy as np

from . import autofp_ref as R

__all__ = [
    "hessian", "dampen", "inverse_factor", "masks_of", "group_error", "encode_group",
    "best_mask", "allocate_levels", "solve_group_error", "propagate", "gptq_quantize",
    "hessian_weighted_error",
]

GROUP, SUBGROUP = R.GROUP, R.SUBGROUP


def hessian(x):
    """H = X^T X in fp64 for calibration activations X [tokens, K] (reading G1)."""
    x = np.asarray(x, dtype=np.float64)
    return x.T @ x


def dampen(h, lam=0.01):
    """H_d = H + lam * mean(diag H) * I (reading G1)."""
    h = np.asarray(h, dtype=np.float64)
    return h + lam * np.mean(np.diag(h)) * np.eye(h.shape[0])


def inverse_factor(h_d):
    """U, upper triangular with a positive diagonal, with H_d^-1 = U^T U
    (reading G1): the Cholesky factor of the inverse."""
    inv = np.linalg.inv(np.asarray(h_d, dtype=np.float64))
    inv = 0.5 * (inv + inv.T)
    return np.linalg.cholesky(inv).T.copy()


def masks_of(level):
    """M_l: the masks refining ``level`` of a group's four subgroups, as bit
    masks, in lexicographic order of their subgroup indices (reading G5)."""
    return [sum(1 << s for s in c) for c in itertools.combinations(range(4), level)]


def _select(mask, w4, wr):
    """What(m) of a group: the refined values on the subgroups of m."""
    sel = np.repeat([(mask >> s) & 1 for s in range(4)], SUBGROUP).astype(bool)
    return np.where(sel[None, :], wr, w4)


def group_error(w_j, w4, wr, h_j, mask):
    """Eq. 7: E_j(m) = sum_i H_ii ||W[:, i] - What[:, i](m)||^2 over the
    group's 16 columns (fp64)."""
    diff = np.asarray(w_j, np.float64) - _select(mask, w4, wr)
    return float(np.dot(np.asarray(h_j, np.float64), np.sum(diff * diff, axis=0)))


def encode_group(w_j, tensor_amax):
    """Lines 15-19 for one group from its current (fp64) weights, reading G4:
    returns (codes [N, 16], scales [N], d [N, 16], W4 = T B q, Wr = T B (q + d/8))."""
    x32 = np.asarray(w_j, dtype=np.float64).astype(np.float32)
    base = R.nvfp4_quantize(x32, tensor_amax=tensor_amax)
    d = R.offset_select(base.v.astype(np.float64) - R.e2m1_value(base.codes))
    tb = np.float64(base.T) * R.e4m3_value(base.scales)            # [N, 1], exact
    s = np.repeat(tb, GROUP, axis=1)
    q = R.e2m1_value(base.codes)
    return base.codes, base.scales[:, 0], d, s * q, s * (q + d / 8.0)


def best_mask(w_j, w4, wr, h_j, level):
    """argmin over M_level of E_j (line 20; first minimum, reading G5)."""
    best, best_e = 0, None
    for m in masks_of(level):
        e = group_error(w_j, w4, wr, h_j, m)
        if best_e is None or e < best_e:
            best, best_e = m, e
    return best


def allocate_levels(w, h_diag, rho=0.2):
    """Lines 4-12: the number of refined subgroups l_j of every group, from
    the original weights. Returns (levels [K/16] int, T)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    G = K // GROUP
    amax = np.max(np.abs(w))
    w64 = w.astype(np.float64)
    h = np.asarray(h_diag, dtype=np.float64)
    L = np.zeros((G, 3))
    for j in range(G):
        J = slice(GROUP * j, GROUP * (j + 1))
        _, _, _, w4, wr = encode_group(w64[:, J], amax)
        for lv in range(3):
            L[j, lv] = min(group_error(w64[:, J], w4, wr, h[J], m) for m in masks_of(lv))
    levels = np.zeros(G, dtype=np.int64)
    budget = min(int(math.floor(rho * K / 4)), 2 * G)
    for _ in range(budget):
        best_j, best_gain = -1, None
        for j in range(G):
            if levels[j] < 2:
                gain = L[j, levels[j]] - L[j, levels[j] + 1]
                if best_gain is None or gain > best_gain:
                    best_j, best_gain = j, gain
        levels[best_j] += 1
    return levels, np.float32(amax) / np.float32(6 * 448)


def solve_group_error(r, u_jj):
    """Line 22: E with E U_JJ = r (U_JJ upper triangular), by forward
    substitution in column order (reading G4). r [N, 16] -> E [N, 16]."""
    r = np.asarray(r, dtype=np.float64)
    e = np.zeros_like(r)
    for i in range(r.shape[1]):
        acc = r[:, i].copy()
        for k in range(i):
            acc = acc - e[:, k] * u_jj[k, i]
        e[:, i] = acc / u_jj[i, i]
    return e


def propagate(w, e, u, j):
    """Line 23: W[:, (j+1)G:] -= E U[J, (j+1)G:], each element's 16-term sum
    accumulated in index order (reading G4). Returns the updated copy."""
    w = np.array(w, dtype=np.float64)
    c0 = GROUP * (j + 1)
    if c0 >= w.shape[1]:
        return w
    rows = u[GROUP * j:GROUP * (j + 1), c0:]
    upd = e[:, 0:1] * rows[0:1, :]
    for i in range(1, GROUP):
        upd = upd + e[:, i:i + 1] * rows[i:i + 1, :]
    w[:, c0:] = w[:, c0:] - upd
    return w


def gptq_quantize(w, u, h_diag, rho=0.2):
    """Algorithm 1 on a weight W [N, K] (fp32) with the inverse-Hessian factor
    U [K, K] and the Hessian diagonal h_diag [K]. Returns the packed tensor as
    ``autofp_ref.quantize_weight`` does (codes, scales, T, mask, offsets,
    n_refined, mask_bits, d) plus ``levels`` (l_j) and ``What`` [N, K] fp64."""
    w = np.asarray(w, dtype=np.float32)
    u = np.asarray(u, dtype=np.float64)
    h = np.asarray(h_diag, dtype=np.float64)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 16")
    G = K // GROUP
    levels, T = allocate_levels(w, h, rho)
    amax = np.max(np.abs(w))
    W = w.astype(np.float64)
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, G), dtype=np.uint8)
    dall = np.zeros((N, K), dtype=np.int8)
    bits = np.zeros(G, dtype=np.uint8)
    what = np.zeros((N, K), dtype=np.float64)
    for j in range(G):
        J = slice(GROUP * j, GROUP * (j + 1))
        q, b, d, w4, wr = encode_group(W[:, J], amax)
        m = best_mask(W[:, J], w4, wr, h[J], int(levels[j]))
        qj = _select(m, w4, wr)
        codes[:, J], scales[:, j], bits[j] = q, b, m
        sel = np.repeat([(m >> s) & 1 for s in range(4)], SUBGROUP).astype(bool)
        dall[:, J] = np.where(sel[None, :], d, 0)
        what[:, J] = qj
        e = solve_group_error(W[:, J] - qj, u[J, J])
        W = propagate(W, e, u, j)
    sel_sg = ((bits.astype(np.int64)[:, None] >> np.arange(4)[None, :]) & 1).astype(bool).reshape(-1)
    per_sg = R.pack_offsets_byte(dall.reshape(N, K // SUBGROUP, SUBGROUP))
    return dict(codes=R.pack_nibbles(codes), scales=scales, T=np.float32(T), q=codes, rows=N, k=K,
                mask=R.pack_nibbles(bits), offsets=np.ascontiguousarray(per_sg[:, sel_sg]),
                n_refined=int(sel_sg.sum()), mask_bits=bits, d=dall, levels=levels, What=what)


def hessian_weighted_error(w, what, h_d):
    """The calibration objective: tr((W - What) H_d (W - What)^T) (fp64)."""
    diff = np.asarray(w, np.float64) - np.asarray(what, np.float64)
    return float(np.einsum("nk,kl,nl->", diff, np.asarray(h_d, np.float64), diff))
