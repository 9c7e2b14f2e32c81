"""Plain CPU reference of AutoFP encode/decode, the AutoFP linear layer and the
two runtime-policy signals.

TEST INFRASTRUCTURE: imported only by the tests, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg. It shares no code with the HIP library.

Paper: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
Exponent-Mantissa Refinement" (arXiv 2611.10165v1), cited below as [AE] with the
section, equation, table or figure.

Precision rules of this oracle:
  * Steps the paper states as floating-point format conversions (Eqs. 2-3) are
    evaluated in IEEE fp32 (``np.float32`` arithmetic: correctly rounded, no
    fused multiply-add), in the order the equations write them.
  * Rounding to E2M1 / E4M3 compares the fp32 input against the exact grid in
    fp64, where every grid value and midpoint is exact.
  * Decoded values and the matrix product are fp64.

Readings taken where the paper leaves a step open are listed in the docstring of
the function that takes them.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(worked examples, closed forms, exhaustive codecs, brute force) except where a
docstring says "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "GROUP", "SUBGROUP", "DEFAULTS", "NVFP4",
    "e2m1_value", "e2m1_encode", "e4m3_value", "e4m3_encode",
    "offset_select", "autofp2_digit",
    "nvfp4_quantize", "activation_refinement", "weight_subgroup_gains",
    "greedy_weight_mask", "weight_offsets",
    "pack_nibbles", "pack_offsets_byte", "unpack_nibbles",
    "quantize_activation", "quantize_weight", "select_weight_mask",
    "decode_activation", "decode_weight", "linear",
    "topk_entropy", "update_norm", "PolicyState", "policy_prefill", "policy_decode_step",
    "silu", "epilogue", "RMS_EPS", "rmsnorm_residual",
]

# [AE] App. B.1: 16 contiguous elements along the reduction dimension share one
# E4M3 group scale.  [AE] §3.2: a group holds four 4-element subgroups (SG = 4,
# §5.1 hyperparameters).
GROUP = 16
SUBGROUP = 4

# [AE] §5.1 "Hyperparameters".  eps of Eq. 1 is not given in the paper
# (reading: 1e-6).
DEFAULTS = dict(
    rho=0.2,               # weight refinement budget
    act_nmse_thresh=0.003,  # activation subgroup refinement threshold
    c2=2.0,                # AutoFP2 scale multiple c (App. B.4, Eq. 4)
    top_k=10,              # G_E top-K
    eps=1e-6,              # L_A stability term (Eq. 1)
    tau=0.10,              # entropy threshold separating decode regimes
    alpha=4, beta=2, n_p=2,  # trend lengths of Table 1
    lambda_d=0.7,          # decode metric weight (Table 1)
)


# ----------------------------------------------------------------------------
# Element and scale codecs
# ----------------------------------------------------------------------------

def e2m1_value(code):
    """Value of a 4-bit E2M1 code ``s e1 e0 m`` (bit 3 = sign).

    [AE] App. B, Table 5 and Table 6: layout 1/2/1, exponent bias 1. Exponent
    field 0 is subnormal (0.5*m); otherwise 2^(e-1) * (1 + m/2). Table 7 prints
    codes in the same ``s e1e0 m`` order (e.g. 3.0 = 0 10 1).
    """
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, (e - 1)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def _rne_on_grid(x, grid):
    """Index of the nearest value of the increasing ``grid`` to each ``x``
    (both exact in fp64); a tie goes to the even index (even mantissa, since
    index = code)."""
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left")
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    dlo = np.abs(x - grid[lo])
    dhi = np.abs(grid[hi] - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


_E2M1_GRID = e2m1_value(np.arange(8))      # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(v):
    """Q_E2M1 of [AE] App. B.1 (Eq. 3): round to the nearest E2M1 value, ties to
    even; magnitudes above 6 saturate to 6 (the format has no infinity).

    Reading (zero sign): a result of magnitude 0 is the canonical +0 code 0x0;
    Table 7 writes 0.00 as ``0 00 0``.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 6.0)
    idx = _rne_on_grid(mag, _E2M1_GRID)
    sign = (v < 0) & (idx != 0)
    return (idx | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e4m3_value(code):
    """Value of an 8-bit E4M3 code (OCP E4M3FN: bias 7, subnormals m/8*2^-6,
    max 448 = 0x7E, codes 0x7F/0xFF are NaN).  [AE] Table 5: E4M3 scale,
    layout 1/4/3, range 2^-9 .. 448."""
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


_E4M3_GRID = e4m3_value(np.arange(0x7F))     # 0 .. 448, increasing


def e4m3_encode(b):
    """Q_E4M3 of [AE] App. B.1 (Eq. 3) for a non-negative group-scale ratio:
    nearest E4M3 value, ties to even, saturating at 448 (no NaN produced)."""
    b = np.asarray(b, dtype=np.float64)
    if np.any(b < 0) or np.any(np.isnan(b)):
        raise ValueError("group scale ratio must be a non-negative number")
    idx = _rne_on_grid(np.minimum(b, 448.0), _E4M3_GRID)
    return idx.astype(np.uint8)


def offset_select(r):
    """Signed offset d in {-2,-1,0,+1} for a residual r = x/(T B) - q.

    [AE] §3.2 and App. E (Alg. 1, the delta step): delta = d * 2^-3 is the
    argmin over D = {-1/4, -1/8, 0, +1/8} of |x/(TB) - q - delta|; "a refinement
    is set to 0 if it would move the element farther".

    Reading (ties): a tie goes to the candidate of smaller |d|, tried in the
    order 0, +1, -1, -2 (the paper does not say; any tie is equally correct).
    """
    r = np.asarray(r, dtype=np.float64)
    cands = np.array([0, 1, -1, -2], dtype=np.int64)
    dist = np.abs(r[..., None] - cands / 8.0)
    return cands[np.argmin(dist, axis=-1)].astype(np.int8)


def autofp2_digit(code):
    """Quinary AutoFP2 digit Q from an E2M1 code.  [AE] §3.2 "AutoFP2": keep the
    sign bit and remap the two exponent bits e1 e0 to a 2-bit magnitude
    {e1 AND e0, e1 XOR e0}; App. B.4: digit 1 absorbs {1, 1.5, 2, 3}."""
    code = np.asarray(code, dtype=np.int64)
    e1 = (code >> 2) & 1
    e0 = (code >> 1) & 1
    mag = 2 * (e1 & e0) + (e1 ^ e0)
    return np.where((code >> 3) & 1, -mag, mag).astype(np.int64)


# ----------------------------------------------------------------------------
# NVFP4 base quantization (Eqs. 2-3)
# ----------------------------------------------------------------------------

@dataclass
class NVFP4:
    codes: np.ndarray    # [rows, K] uint8, one E2M1 code per element
    scales: np.ndarray   # [rows, K/16] uint8 E4M3 group scales B
    T: np.float32        # per-tensor fp32 scale
    v: np.ndarray        # [rows, K] fp32 normalized values x / (T B)
    s: np.ndarray        # [rows, K/16] fp32 T * B as rounded for the division


def nvfp4_quantize(x, tensor_amax=None):
    """NVFP4 quantization, [AE] App. B.1, Eqs. 2-3, evaluated in fp32.

        T   = amax(X) / (6*448)
        B_j = Q_E4M3(amax(X_j) / (6 T))
        q_i = Q_E2M1(x_i / (T B_j))

    Reading (operation order): the products in the denominators are formed
    first, each rounded to fp32: ``sixT = 6*T``; ``b = a_j / sixT``;
    ``s = T * B``; ``v = x / s``. When 6T or s is zero the group encodes to
    zeros (B = 0, all codes +0).

    ``tensor_amax`` replaces amax(X) when ``x`` holds only some rows of a
    larger tensor (the per-tensor scale is a property of the whole tensor).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % GROUP:
        raise ValueError("x must be [rows, K] with K a multiple of 16")
    rows, K = x.shape
    G = K // GROUP
    if tensor_amax is None:
        amax = np.max(np.abs(x)) if x.size else np.float32(0)
    else:
        amax = np.float32(tensor_amax)
    T = np.float32(amax) / np.float32(6 * 448)
    six_t = np.float32(6.0) * T
    a = np.max(np.abs(x.reshape(rows, G, GROUP)), axis=2) if x.size else np.zeros((rows, G), np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        b = (a / six_t) if six_t > 0 else np.zeros_like(a)
    B = e4m3_encode(b)
    s = (T * e4m3_value(B).astype(np.float32)).astype(np.float32)
    s_el = np.repeat(s, GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s_el != 0, x / np.where(s_el != 0, s_el, np.float32(1)), np.float32(0))
    v = v.astype(np.float32)
    q = e2m1_encode(v)
    return NVFP4(codes=q, scales=B, T=np.float32(T), v=v, s=s)


def _residual(base: NVFP4):
    """r = v - q in fp64 (the fp32 subtraction is exact here: q is the E2M1
    value nearest to v, so v and q lie within a factor of two or q = 0)."""
    return base.v.astype(np.float64) - e2m1_value(base.codes)


# ----------------------------------------------------------------------------
# AutoFP6 refinement
# ----------------------------------------------------------------------------

def activation_refinement(base: NVFP4, exclude_bits=None, thresh=0.003):
    """Activation mask M_A and offsets d.

    [AE] §6.4 (PPU) and §5.1: compute each subgroup's NMSE and refine the
    subgroups whose NMSE is above the threshold (0.003), excluding those in the
    weight mask M_W; offsets d as in ``offset_select``. [AE] §2.3 / Fig. 5 fix
    NMSE as sum((x - xq)^2) / sum(x^2) over the subgroup.

    Readings: NMSE is taken on the normalized values v = x/(TB) (the ratio is
    scale-free); in fp32, ``num = ((e0^2 + e1^2) + e2^2) + e3^2`` with
    e_i = v_i - q_i, ``den`` alike on v_i, and the test is ``den > 0 and
    num > thresh * den`` (fp32 products, no fused multiply-add).

    Returns (mask_bits [rows, K/16] uint8 with bit k = SG k, d [rows, K] int8
    with d = 0 outside refined subgroups).
    """
    rows, K = base.codes.shape
    nsg = K // SUBGROUP
    v = base.v.reshape(rows, nsg, SUBGROUP).astype(np.float32)
    e = (base.v - e2m1_value(base.codes).astype(np.float32)).astype(np.float32)
    e = e.reshape(rows, nsg, SUBGROUP)
    num = ((e[..., 0] * e[..., 0] + e[..., 1] * e[..., 1]) + e[..., 2] * e[..., 2]) + e[..., 3] * e[..., 3]
    den = ((v[..., 0] * v[..., 0] + v[..., 1] * v[..., 1]) + v[..., 2] * v[..., 2]) + v[..., 3] * v[..., 3]
    refine = (den > 0) & (num > np.float32(thresh) * den)
    refine = refine.reshape(rows, K // GROUP, 4)
    if exclude_bits is not None:
        ex = np.asarray(exclude_bits, dtype=np.int64)
        ex_sg = ((ex[:, None] >> np.arange(4)[None, :]) & 1).astype(bool)  # [G, 4]
        refine &= ~ex_sg[None, :, :]
    mask_bits = (refine * (1 << np.arange(4))).sum(axis=2).astype(np.uint8)
    d_all = offset_select(_residual(base)).reshape(rows, K // GROUP, 4, SUBGROUP)
    d = np.where(refine[..., None], d_all, 0).reshape(rows, K).astype(np.int8)
    return mask_bits, d


def weight_subgroup_gains(w, base: NVFP4):
    """Per-row, per-subgroup reduction in squared error from refining it.

    [AE] App. E (Alg. 1): E_j(m) is the error of group j with the refined
    values on the subgroups of m; with the identity Hessian (no calibration
    data; reading) the error is additive over subgroups, so the reduction from
    refining subgroup k of group j in row n is
        g[n, j, k] = sum_i (eb_i^2 - er_i^2),
        eb = w - T B q,   er = w - T B (q + d/8)
    with the dequantized values of Alg. 1 (T B q and T B (q + delta), exact in
    fp64).  Evaluated in fp64: per element ``eb*eb - er*er``, then summed over
    the four elements left to right.  Returns g [rows, K/4] fp64 (>= 0).
    """
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, K = w.shape
    tb = np.float64(base.T) * e4m3_value(base.scales)        # exact product
    s = np.repeat(tb, GROUP, axis=1)
    q = e2m1_value(base.codes)
    d = offset_select(_residual(base)).astype(np.float64)
    eb = w - s * q
    er = w - s * (q + d / 8.0)
    ge = (eb * eb - er * er).reshape(rows, K // SUBGROUP, SUBGROUP)
    return ((ge[..., 0] + ge[..., 1]) + ge[..., 2]) + ge[..., 3]


def greedy_weight_mask(col_gain, budget):
    """Budget allocation of [AE] App. E, Alg. 1 (allocation loop): start every
    group at l_j = 0 refined subgroups; ``budget`` times, give one more refined
    subgroup to the group with the largest marginal reduction
    L_j(l_j) - L_j(l_j + 1) among groups with l_j < 2 (first such group on a
    tie).  With additive errors L_j(l) - L_j(l+1) is the (l+1)-th largest
    subgroup gain of group j.

    Reading (ties inside a group): equal gains rank the lower subgroup first.
    ``col_gain`` is [G, 4] (gain per group and subgroup summed over rows).
    Returns mask bits [G] uint8 (bit k = SG k).
    """
    col_gain = np.asarray(col_gain, dtype=np.float64)
    G = col_gain.shape[0]
    order = np.argsort(-col_gain, axis=1, kind="stable")     # per group, best first
    ranked = np.take_along_axis(col_gain, order, axis=1)
    level = np.zeros(G, dtype=np.int64)
    for _ in range(int(budget)):
        live = level < 2
        if not live.any():
            break
        marg = np.where(live, ranked[np.arange(G), np.minimum(level, 3)], -np.inf)
        j = int(np.argmax(marg))
        level[j] += 1
    bits = np.zeros(G, dtype=np.uint8)
    for j in range(G):
        for t in range(level[j]):
            bits[j] |= np.uint8(1 << int(order[j, t]))
    return bits


def select_weight_mask(w, rho=0.2):
    """Weight mask M_W for a [N, K] weight: one 4-bit mask per 16-column group,
    shared by every row ([AE] §3.2), with floor(rho * K / 4) refined subgroups
    in total and at most two per group (Alg. 1 allocates l_j in {0, 1, 2}).

    Reading (cross-row sum): the column gain G[j, k] is the sum over rows
    n = 0 .. N-1 of ``weight_subgroup_gains`` taken in that order in fp64.
    Reading (budget rounding): floor(rho * K / 4), with rho*K/4 formed in fp64.
    Returns (mask_bits [K/16] uint8, R = number of refined subgroups).
    """
    w = np.asarray(w, dtype=np.float32)
    base = nvfp4_quantize(w)
    g = weight_subgroup_gains(w, base)
    col = np.zeros(g.shape[1], dtype=np.float64)
    for n in range(g.shape[0]):
        col = col + g[n]
    budget = int(math.floor(rho * w.shape[1] / 4))
    bits = greedy_weight_mask(col.reshape(-1, 4), budget)
    return bits, int(sum(bin(int(b)).count("1") for b in bits))


def weight_offsets(base: NVFP4, mask_bits):
    """Weight offsets d on the subgroups of M_W ([AE] Alg. 1, delta step), zero
    elsewhere; returns d [N, K] int8."""
    rows, K = base.codes.shape
    d_all = offset_select(_residual(base)).reshape(rows, K // GROUP, 4, SUBGROUP)
    bits = np.asarray(mask_bits, dtype=np.int64)
    sel = ((bits[:, None] >> np.arange(4)[None, :]) & 1).astype(bool)
    return np.where(sel[None, :, :, None], d_all, 0).reshape(rows, K).astype(np.int8)


# ----------------------------------------------------------------------------
# Byte layout (the library's packed format)
# ----------------------------------------------------------------------------

def pack_nibbles(vals):
    """Two 4-bit values per byte, element 2i in the low nibble.  Used for E2M1
    codes ([rows, K] -> [rows, K/2]) and for the 4-bit masks ([.., G] ->
    [.., ceil(G/2)], group 2i in the low nibble; [AE] Fig. 23 packs two group
    masks per byte)."""
    vals = np.asarray(vals, dtype=np.uint8)
    if vals.shape[-1] % 2:
        vals = np.concatenate([vals, np.zeros(vals.shape[:-1] + (1,), np.uint8)], axis=-1)
    return (vals[..., 0::2] & 0xF) | ((vals[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed, n):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out[..., :n]


def pack_offsets_byte(d4):
    """One byte per subgroup: the four 2-bit two's-complement offsets, element k
    of the subgroup in bits [2k+1:2k].  [AE] Fig. 23 / Table 7 fix the codes
    (+1 = 01, 0 = 00, -1 = 11, -2 = 10)."""
    d4 = np.asarray(d4, dtype=np.int64) & 3
    return (d4[..., 0] | (d4[..., 1] << 2) | (d4[..., 2] << 4) | (d4[..., 3] << 6)).astype(np.uint8)


def _mask_bits_of(packed_mask, G):
    return unpack_nibbles(packed_mask, G)


# ----------------------------------------------------------------------------
# Public quantizers producing the packed format
# ----------------------------------------------------------------------------

def quantize_activation(x, refine=False, exclude_mask=None, thresh=0.003, tensor_amax=None):
    """Encode activations X [B, K] (fp32, or bf16 widened exactly by the caller)
    to AutoFP: NVFP4 base with one per-tensor scale over the whole call
    ([AE] App. B.1; reading: one T over all rows of the call), plus, when
    ``refine``, the activation mask (excluding the packed weight mask
    ``exclude_mask`` [K/32]) and dense offsets [B, K/4] (one byte per subgroup,
    0x00 where not refined)."""
    base = nvfp4_quantize(x, tensor_amax)
    rows, K = base.codes.shape
    out = dict(codes=pack_nibbles(base.codes), scales=base.scales.copy(), T=base.T,
               q=base.codes, rows=rows, k=K)
    if refine:
        ex = None if exclude_mask is None else _mask_bits_of(exclude_mask, K // GROUP)
        bits, d = activation_refinement(base, ex, thresh)
        out["mask"] = pack_nibbles(bits)
        out["offsets"] = pack_offsets_byte(d.reshape(rows, K // SUBGROUP, SUBGROUP))
        out["mask_bits"] = bits
        out["d"] = d
    return out


def quantize_weight(w, mask=None, tensor_amax=None):
    """Encode a weight W [N, K] (fp32): NVFP4 base; with a packed weight mask
    [K/32] also the compacted offsets [N, R]: for every row, one byte per
    refined subgroup in ascending (group, subgroup) order ([AE] §4 stores the
    signed offsets of each refined subgroup in a byte of their own; Fig. 23)."""
    base = nvfp4_quantize(w, tensor_amax)
    N, K = base.codes.shape
    out = dict(codes=pack_nibbles(base.codes), scales=base.scales.copy(), T=base.T,
               q=base.codes, rows=N, k=K)
    if mask is not None:
        bits = _mask_bits_of(mask, K // GROUP)
        d = weight_offsets(base, bits)
        sel = ((bits.astype(np.int64)[:, None] >> np.arange(4)[None, :]) & 1).astype(bool).reshape(-1)
        per_sg = pack_offsets_byte(d.reshape(N, K // SUBGROUP, SUBGROUP))
        out["mask"] = np.asarray(mask, dtype=np.uint8).copy()
        out["offsets"] = np.ascontiguousarray(per_sg[:, sel])
        out["n_refined"] = int(sel.sum())
        out["mask_bits"] = bits
        out["d"] = d
    return out


# ----------------------------------------------------------------------------
# Decode (dequantized operands, fp64) and the linear layer
# ----------------------------------------------------------------------------

def _d_from_offsets_dense(offsets, rows, K):
    b = np.asarray(offsets, dtype=np.int64).reshape(rows, K // SUBGROUP)
    d = np.stack([(b >> (2 * k)) & 3 for k in range(4)], axis=-1)
    d = np.where(d >= 2, d - 4, d)
    return d.reshape(rows, K)


def decode_activation(pk, level):
    """X_hat in fp64. Level 4 (and the activation side of level 2, W2A4):
    T * B * q ([AE] Eq. 3). Level 6: T * B * (q + M_A * d/8) ([AE] §3.2,
    X_tilde = X_q + M_X . X_r with the fixed step 2^-3)."""
    rows, K = pk["rows"], pk["k"]
    q = e2m1_value(unpack_nibbles(pk["codes"], K))
    s = float(pk["T"]) * np.repeat(e4m3_value(pk["scales"]), GROUP, axis=1)
    if level == 6:
        q = q + _d_from_offsets_dense(pk["offsets"], rows, K) / 8.0
    elif level not in (2, 4):
        raise ValueError("level must be 2, 4 or 6")
    return s * q


def decode_weight(pk, level, c2=2.0):
    """W_hat in fp64. Level 4: T B q. Level 6: T B (q + M_W d/8) from the
    compacted offsets. Level 2: c T B Q with Q the AutoFP2 digit ([AE] App. B.4,
    Eq. 4)."""
    N, K = pk["rows"], pk["k"]
    codes = unpack_nibbles(pk["codes"], K)
    s = float(pk["T"]) * np.repeat(e4m3_value(pk["scales"]), GROUP, axis=1)
    if level == 4:
        return s * e2m1_value(codes)
    if level == 2:
        return c2 * s * autofp2_digit(codes).astype(np.float64)
    if level != 6:
        raise ValueError("level must be 2, 4 or 6")
    bits = _mask_bits_of(pk["mask"], K // GROUP).astype(np.int64)
    sel = ((bits[:, None] >> np.arange(4)[None, :]) & 1).astype(bool).reshape(-1)
    offs = np.asarray(pk["offsets"], dtype=np.int64).reshape(N, -1)
    if offs.shape[1] != sel.sum():
        raise ValueError("offsets do not match the mask")
    dense = np.zeros((N, K // SUBGROUP), dtype=np.int64)
    dense[:, sel] = offs
    d = _d_from_offsets_dense(dense, N, K)
    return s * (e2m1_value(codes) + d / 8.0)


def linear(wpk, xpk, level, c2=2.0):
    """Y = X_hat . W_hat^T in fp64 at one precision level ([AE] §3.1: each layer
    runs WxAx-KVx, x in {2,4,6}, with the 2-bit level on weights only, W2A4;
    §3.2: the refined GEMM is the product of the refined operands)."""
    a_level = 4 if level == 2 else level
    X = decode_activation(xpk, a_level)
    W = decode_weight(wpk, level, c2)
    return X @ W.T


# ----------------------------------------------------------------------------
# Producer epilogue (the layer's elementwise step before the next encode)
# ----------------------------------------------------------------------------

def silu(g):
    """silu(g) = g / (1 + e^-g) = g * sigmoid(g), fp64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def epilogue(op, z, k, residual=None):
    """The elementwise step the post-processing unit applies to a completed
    linear output before quantizing it into the next layer's activation
    ([AE] §6.4: the PPU quantizes completed outputs into the next layer's
    input activations and performs the non-linear operations). fp64:
      "copy"     v = z[:, :k]
      "residual" v = residual + z[:, :k]
      "swiglu"   v = silu(z[:, :k]) * z[:, k:2k]
      "residual_rmsnorm"  v = RMSNorm(residual + z[:, :k]) (rmsnorm_residual)
    Reading: the pages name no model; these are the residual stream and the
    gated MLP of the Llama-shaped layers the workloads use."""
    z = np.asarray(z, dtype=np.float64)
    if op == "copy":
        return z[:, :k].copy()
    if op == "residual":
        return np.asarray(residual, dtype=np.float64) + z[:, :k]
    if op == "swiglu":
        return silu(z[:, :k]) * z[:, k:2 * k]
    if op == "residual_rmsnorm":
        return rmsnorm_residual(z, k, residual)[0].astype(np.float64)
    raise ValueError(op)


RMS_EPS = 1e-5   # RMSNorm epsilon of the Llama-3 layers the workloads are shaped after


def rmsnorm_residual(z, k, residual, eps=RMS_EPS):
    """The residual add of a pre-norm block followed by the RMSNorm that
    forms the next linear layer's input, as one post-processing step ([AE]
    §6.4: the PPU turns completed outputs into the next layer's input
    activations, non-linear operations included):
      u = residual + z[:, :k]                  (the new hidden state; fp32, as an fp32 sum)
      c = 1 / sqrt(sum_j u_j^2 / k + eps)      (per row; the squares summed in fp64, c rounded to fp32)
      v = u * c                                (one fp32 product per element)
    Reading: the pages name no model; RMSNorm with unit gain and Llama-3's
    eps = 1e-5. The squares of fp32 values are exact in fp64, so the row sum
    is fixed up to fp64 rounding and c to its fp32 rounding. Returns (v, u),
    both fp32."""
    z = np.asarray(z, dtype=np.float64)
    u = (np.asarray(residual, dtype=np.float64) + z[:, :k]).astype(np.float32)
    u64 = u.astype(np.float64)
    c = (1.0 / np.sqrt(np.sum(u64 * u64, axis=1) / k + eps)).astype(np.float32)
    v = u * c[:, None]          # float32 x float32 -> float32, round to nearest even
    return v.astype(np.float32), u


# ----------------------------------------------------------------------------
# Runtime policy signals and rules
# ----------------------------------------------------------------------------

def topk_entropy(logits, k=10):
    """G_E: normalized Shannon entropy of the top-K next-token logits
    ([AE] §3.1 and App. D.1): softmax over the K largest logits of each row,
    H = -sum p ln p, divided by ln K (K = 10, §5.1).  With k >= V the whole
    vocabulary is used (ln V).  Reading: raw logits (no temperature)."""
    z = np.asarray(logits, dtype=np.float64)
    if z.ndim == 1:
        z = z[None, :]
    V = z.shape[1]
    kk = min(int(k), V)
    out = np.zeros(z.shape[0])
    for b in range(z.shape[0]):
        top = np.sort(z[b])[V - kk:]
        t = top - top.max()
        p = np.exp(t)
        p /= p.sum()
        nz = p[p > 0]
        h = float(-(nz * np.log(nz)).sum())
        out[b] = h / math.log(kk) if kk > 1 else 0.0
    return out


def update_norm(h_prev, h_cur, eps=1e-6):
    """L_A of [AE] Eq. 1 per row: ||H_l - H_(l-1)||_2 / (||H_(l-1)||_2 + eps)."""
    hp = np.asarray(h_prev, dtype=np.float64)
    hc = np.asarray(h_cur, dtype=np.float64)
    if hp.ndim == 1:
        hp, hc = hp[None], hc[None]
    num = np.sqrt(((hc - hp) ** 2).sum(axis=1))
    den = np.sqrt((hp ** 2).sum(axis=1)) + eps
    return num / den


@dataclass
class PolicyState:
    """Running statistics of the metric M for one sequence and phase.

    Reading: mu and sigma are the running mean and population standard
    deviation of every earlier M value of the sequence in the current phase
    (prefill, or the decode steps so far), excluding the value being judged.
    Parity unpinned against the paper beyond the hand-built sequences of the
    tests (its layer traces are figures).
    """
    count: int = 0
    mean: float = 0.0
    m2: float = 0.0
    history: list = field(default_factory=list)

    def add(self, m):
        self.count += 1
        delta = m - self.mean
        self.mean += delta / self.count
        self.m2 += delta * (m - self.mean)
        self.history.append(m)

    @property
    def std(self):
        return math.sqrt(self.m2 / self.count) if self.count else 0.0


def _trend(counters, m, mu):
    if m > mu:
        counters[0] += 1
        counters[1] = 0
    elif m < mu:
        counters[1] += 1
        counters[0] = 0
    else:
        counters[0] = counters[1] = 0


def policy_prefill(l_a, state=None, n_p=2):
    """Prefill precision per layer from M_P = L_A ([AE] §3.1 "Prefill policy",
    Table 1). Layers up to and including the first spike (M > mu + 3 sigma,
    needing at least two earlier values) run at 6 bits; after it, n_p
    consecutive layers below (above) mu lower (raise) the next layer by one
    level of P = {2, 4, 6}, saturating.  Returns the bits of every layer."""
    st = state or PolicyState()
    bits, p, spike, cnt = [], 6, False, [0, 0]
    for m in map(float, l_a):
        bits.append(p)
        if not spike:
            if st.count >= 2 and m > st.mean + 3.0 * st.std:
                spike = True
        else:
            _trend(cnt, m, st.mean)
            if cnt[0] >= n_p:
                p, cnt[0] = min(6, p + 2), 0
            elif cnt[1] >= n_p:
                p, cnt[1] = max(2, p - 2), 0
        st.add(m)
    return bits


def policy_decode_step(l_a, g_prev, state, tau=0.10, alpha=4, beta=2, lam=0.7):
    """Decode precision per layer for one step ([AE] §3.1 "Decode policy",
    Table 1): M_D = lam L_A + (1 - lam) G_E with the previous step's G_E; layer 0
    starts at 4 bits; at a high-entropy step (G_E >= tau) beta consecutive layers
    above mu raise and alpha consecutive layers below mu lower the next layer;
    at a low-entropy step alpha and beta swap.  Reading: the consecutive-layer
    counters restart at every step; ``state`` carries mu over the decode
    steps.  Returns the bits of every layer."""
    high = g_prev >= tau
    n_up, n_down = (beta, alpha) if high else (alpha, beta)
    bits, p, cnt = [], 4, [0, 0]
    for la in map(float, l_a):
        bits.append(p)
        m = lam * la + (1.0 - lam) * float(g_prev)
        if state.count:
            _trend(cnt, m, state.mean)
            if cnt[0] >= n_up:
                p, cnt[0] = min(6, p + 2), 0
            elif cnt[1] >= n_down:
                p, cnt[1] = max(2, p - 2), 0
        state.add(m)
    return bits
