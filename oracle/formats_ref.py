"""Plain CPU reference of the AutoFP format variants: AutoFP8 (4-bit signed
offsets), the exponent-scaled offset step, and the FP6g comparator format.

TEST INFRASTRUCTURE: imported only by the tests, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg. It shares no code with the HIP library.

Paper: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
Exponent-Mantissa Refinement" (arXiv 2611.10165v1), cited as [AE]:
  * App. I "Extension to 8 bits" and Table 10: widening the signed offsets from
    2 to 4 bits gives AutoFP8, stored at 5.3 bits per weight (rho = 0.2).
  * §6.5 "Refinement Decoding" and Fig. 14(a): the fixed offset step 2^-3
    against the exact, per-element exponent step 2^(e-3).
  * App. B.2: FP6g, the group-scaled 6-bit baseline: NVFP4's group size and
    scaling hierarchy with E2M3 elements (bias 1, maximum 7.5) in place of E2M1.

Precision rules are those of ``autofp_ref``: format conversions in IEEE fp32 in
the written order, grid rounding against exact fp64 grids, decoded values and
products in fp64.

Offset formats (the ``fmt`` argument):
  "autofp6"  : d in {-2,-1,0,+1}, delta = d * 2^-3 (the default of autofp_ref)
  "autofp6e" : d in {-2,-1,0,+1}, delta = d * 2^(e-3), e the unbiased exponent
               of the element's E2M1 value q (0 for the subnormal codes)
  "autofp8"  : d in {-8,...,+7}, delta = d * 2^-3
Reading (AutoFP8 step): App. I says only that the offsets widen from 2 to 4
bits; the plainest reading keeps the fixed step of §3.2 and Alg. 1 (the set D
is d * 2^-3) and widens the range of d. A consequence used by the library: the
2-bit offset of an element is the 4-bit one clamped to [-2, +1] (both are the
argmin of |r - d/8| over a range of integers), so an AutoFP8 tensor also runs
at level 6, as Table 10's P = {2, 4, 6, 8} at one storage of 5.3 bits requires.

Parity status: every function is pinned by ``tests/test_oracle_formats.py``
(Table 6 grid, Table 10 storage, brute force with exact rationals, reduction to
the AutoFP6 case, the clamp identity).
"""

from __future__ import annotations

import numpy as np

from . import autofp_ref as R

__all__ = [
    "FORMATS", "e2m3_value", "e2m3_encode", "offset_candidates", "offset_select_fmt", "delta_of", "step_of",
    "quantize_activation_fmt", "quantize_weight_fmt", "select_weight_mask_fmt",
    "decode_activation_fmt", "decode_weight_fmt", "linear_fmt",
    "fp6g_quantize", "pack_fp6", "unpack_fp6", "decode_fp6g", "linear_fp6g",
    "pack_offsets_word", "storage_bits_per_weight",
]

FORMATS = ("autofp6", "autofp6e", "autofp8")
GROUP, SUBGROUP = R.GROUP, R.SUBGROUP


# ----------------------------------------------------------------------------
# Offsets
# ----------------------------------------------------------------------------

def offset_candidates(fmt):
    """Signed offsets d of a format, in tie-break order: smaller |d| first,
    then the positive one (only r = 0 ties two of equal |d|, where 0 wins)."""
    if fmt in ("autofp6", "autofp6e"):
        return np.array([0, 1, -1, -2], dtype=np.int64)
    if fmt == "autofp8":
        c = [0]
        for m in range(1, 9):
            if m <= 7:
                c.append(m)
            c.append(-m)
        return np.array(c, dtype=np.int64)
    raise ValueError(f"unknown offset format {fmt}")


def _exponent_of_code(codes):
    """Unbiased exponent e of an E2M1 code's value: field 00 (0, 0.5) and
    01 (1, 1.5) give 0, 10 (2, 3) gives 1, 11 (4, 6) gives 2 ([AE] Table 5:
    bias 1, the subnormal field has the exponent of field 01)."""
    f = (np.asarray(codes, dtype=np.int64) >> 1) & 3
    return np.maximum(f - 1, 0)


def step_of(codes, fmt):
    """Offset step per element: 2^-3, or 2^(e-3) for "autofp6e"."""
    codes = np.asarray(codes, dtype=np.int64)
    if fmt == "autofp6e":
        return np.ldexp(1.0, _exponent_of_code(codes) - 3)
    return np.full(codes.shape, 0.125)


def offset_select_fmt(r, codes, fmt):
    """d = argmin over the format's candidates of |r - d * step| ([AE] Alg. 1,
    the delta step: the refinement nearest to x/(TB) - q; zero when refining
    would move the element farther), ties as in ``offset_candidates``."""
    r = np.asarray(r, dtype=np.float64)
    st = step_of(codes, fmt)
    cands = offset_candidates(fmt)
    dist = np.abs(r[..., None] - cands * st[..., None])
    return cands[np.argmin(dist, axis=-1)].astype(np.int8)


def delta_of(d, codes, fmt, level):
    """Refinement delta of stored offsets d at execution level ``level``:
    d * step, with an AutoFP8 tensor at level 6 using d clamped to [-2, +1]."""
    d = np.asarray(d, dtype=np.float64)
    if fmt == "autofp8" and level == 6:
        d = np.clip(d, -2, 1)
    return d * step_of(codes, fmt)


def pack_offsets_word(d4):
    """AutoFP8 storage: two bytes per subgroup, the four 4-bit two's-complement
    offsets with element k of the subgroup in bits [4k+3:4k] (little-endian:
    elements 0, 1 in the first byte). Returns [..., 2] uint8."""
    d4 = np.asarray(d4, dtype=np.int64) & 15
    w = d4[..., 0] | (d4[..., 1] << 4) | (d4[..., 2] << 8) | (d4[..., 3] << 12)
    return np.stack([w & 0xFF, w >> 8], axis=-1).astype(np.uint8)


def _unpack_offsets(raw, rows, nsg, fmt):
    """d [rows, nsg, 4] from the stored offset bytes of nsg subgroups per row."""
    raw = np.asarray(raw, dtype=np.int64)
    if fmt == "autofp8":
        w = raw.reshape(rows, nsg, 2)
        word = w[..., 0] | (w[..., 1] << 8)
        d = np.stack([(word >> (4 * k)) & 15 for k in range(4)], axis=-1)
        return np.where(d >= 8, d - 16, d)
    b = raw.reshape(rows, nsg)
    d = np.stack([(b >> (2 * k)) & 3 for k in range(4)], axis=-1)
    return np.where(d >= 2, d - 4, d)


def _pack_offsets(d4, fmt):
    if fmt == "autofp8":
        return pack_offsets_word(d4).reshape(d4.shape[0], -1)
    return R.pack_offsets_byte(d4)


def storage_bits_per_weight(fmt, rho=0.2):
    """Stored bits per weight element: 4-bit codes, one 8-bit scale per 16,
    and a fraction rho of the elements with an offset of 2 (AutoFP6) or 4
    (AutoFP8) bits (the 4-bit masks per 16 elements are shared by all rows)."""
    width = 4 if fmt == "autofp8" else 2
    return 4.0 + 8.0 / GROUP + rho * width


# ----------------------------------------------------------------------------
# Quantizers and decode for the offset formats
# ----------------------------------------------------------------------------

def quantize_activation_fmt(x, fmt, refine=False, exclude_mask=None, thresh=0.003, tensor_amax=None):
    """As ``autofp_ref.quantize_activation`` (the mask M_A is the same NMSE
    rule: it depends on the base values only), with the format's offsets;
    AutoFP8 stores two bytes per subgroup ([rows, K/2], dense)."""
    base = R.nvfp4_quantize(x, tensor_amax)
    rows, K = base.codes.shape
    out = dict(codes=R.pack_nibbles(base.codes), scales=base.scales.copy(), T=base.T, q=base.codes,
               rows=rows, k=K, fmt=fmt)
    if refine:
        ex = None if exclude_mask is None else R.unpack_nibbles(exclude_mask, K // GROUP)
        bits, _ = R.activation_refinement(base, ex, thresh)
        r = base.v.astype(np.float64) - R.e2m1_value(base.codes)
        d_all = offset_select_fmt(r, base.codes, fmt)
        sel = ((bits.astype(np.int64)[..., None] >> np.arange(4)) & 1).astype(bool)   # [rows, G, 4]
        d = np.where(np.repeat(sel.reshape(rows, -1), SUBGROUP, axis=1), d_all, 0).astype(np.int8)
        out["mask"] = R.pack_nibbles(bits)
        out["offsets"] = _pack_offsets(d.reshape(rows, K // SUBGROUP, SUBGROUP), fmt)
        out["mask_bits"] = bits
        out["d"] = d
    return out


def weight_subgroup_gains_fmt(w, base, fmt):
    """``autofp_ref.weight_subgroup_gains`` with the format's refinement:
    g = sum over the subgroup of (eb^2 - er^2), eb = w - TBq,
    er = w - TB(q + delta), fp64, left to right."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, K = w.shape
    s = np.repeat(np.float64(base.T) * R.e4m3_value(base.scales), GROUP, axis=1)
    q = R.e2m1_value(base.codes)
    d = offset_select_fmt(base.v.astype(np.float64) - q, base.codes, fmt).astype(np.float64)
    delta = d * step_of(base.codes, fmt)
    eb = w - s * q
    er = w - s * (q + delta)
    ge = (eb * eb - er * er).reshape(rows, K // SUBGROUP, SUBGROUP)
    return ((ge[..., 0] + ge[..., 1]) + ge[..., 2]) + ge[..., 3]


def select_weight_mask_fmt(w, fmt, rho=0.2):
    """``autofp_ref.select_weight_mask`` ([AE] App. E, Alg. 1 allocation with the
    identity Hessian) with the gains of the format's refinement."""
    import math
    w = np.asarray(w, dtype=np.float32)
    base = R.nvfp4_quantize(w)
    g = weight_subgroup_gains_fmt(w, base, fmt)
    col = np.zeros(g.shape[1], dtype=np.float64)
    for n in range(g.shape[0]):
        col = col + g[n]
    bits = R.greedy_weight_mask(col.reshape(-1, 4), int(math.floor(rho * w.shape[1] / 4)))
    return bits, int(sum(bin(int(b)).count("1") for b in bits))


def quantize_weight_fmt(w, fmt, mask=None, tensor_amax=None):
    """As ``autofp_ref.quantize_weight`` with the format's offsets: compacted,
    one byte (AutoFP6) or two (AutoFP8) per refined subgroup in ascending
    (group, subgroup) order."""
    base = R.nvfp4_quantize(w, tensor_amax)
    N, K = base.codes.shape
    out = dict(codes=R.pack_nibbles(base.codes), scales=base.scales.copy(), T=base.T, q=base.codes,
               rows=N, k=K, fmt=fmt)
    if mask is not None:
        bits = R.unpack_nibbles(mask, K // GROUP)
        sel = ((bits.astype(np.int64)[:, None] >> np.arange(4)[None, :]) & 1).astype(bool).reshape(-1)
        r = base.v.astype(np.float64) - R.e2m1_value(base.codes)
        d_all = offset_select_fmt(r, base.codes, fmt)
        d = np.where(np.repeat(sel, SUBGROUP)[None, :], d_all, 0).astype(np.int8)
        per_sg = d.reshape(N, K // SUBGROUP, SUBGROUP)[:, sel]          # [N, R, 4]
        out["mask"] = np.asarray(mask, dtype=np.uint8).copy()
        out["offsets"] = np.ascontiguousarray(_pack_offsets(per_sg, fmt))
        out["n_refined"] = int(sel.sum())
        out["mask_bits"] = bits
        out["d"] = d
    return out


def decode_activation_fmt(pk, level):
    """X_hat in fp64: T B q at levels 2 and 4; T B (q + M_A delta) at 6 and 8."""
    fmt = pk["fmt"]
    rows, K = pk["rows"], pk["k"]
    codes = R.unpack_nibbles(pk["codes"], K)
    s = float(pk["T"]) * np.repeat(R.e4m3_value(pk["scales"]), GROUP, axis=1)
    q = R.e2m1_value(codes)
    if level in (6, 8):
        if level == 8 and fmt != "autofp8":
            raise ValueError("level 8 needs AutoFP8 operands")
        d = _unpack_offsets(pk["offsets"], rows, K // SUBGROUP, fmt).reshape(rows, K)
        q = q + delta_of(d, codes, fmt, level)
    elif level not in (2, 4):
        raise ValueError("level must be 2, 4, 6 or 8")
    return s * q


def decode_weight_fmt(pk, level, c2=2.0):
    """W_hat in fp64: level 2 c T B Q (AutoFP2), 4 T B q, 6 / 8 T B (q + M_W delta)."""
    fmt = pk["fmt"]
    N, K = pk["rows"], pk["k"]
    codes = R.unpack_nibbles(pk["codes"], K)
    s = float(pk["T"]) * np.repeat(R.e4m3_value(pk["scales"]), GROUP, axis=1)
    if level == 4:
        return s * R.e2m1_value(codes)
    if level == 2:
        return c2 * s * R.autofp2_digit(codes).astype(np.float64)
    if level not in (6, 8) or (level == 8 and fmt != "autofp8"):
        raise ValueError("bad level for this format")
    bits = R.unpack_nibbles(pk["mask"], K // GROUP).astype(np.int64)
    sel = ((bits[:, None] >> np.arange(4)[None, :]) & 1).astype(bool).reshape(-1)
    n_ref = int(sel.sum())
    d_ref = _unpack_offsets(pk["offsets"], N, n_ref, fmt)          # [N, n_ref, 4]
    d = np.zeros((N, K // SUBGROUP, SUBGROUP), dtype=np.int64)
    d[:, sel] = d_ref
    d = d.reshape(N, K)
    return s * (R.e2m1_value(codes) + delta_of(d, codes, fmt, level))


def linear_fmt(wpk, xpk, level, c2=2.0):
    """Y = X_hat . W_hat^T in fp64 at one level (2: W2A4; 4: W4A4; 6: W6A6;
    8: W8A8 with AutoFP8 operands)."""
    if wpk["fmt"] != xpk["fmt"]:
        raise ValueError("operands of different offset formats")
    X = decode_activation_fmt(xpk, 4 if level == 2 else level)
    W = decode_weight_fmt(wpk, level, c2)
    return X @ W.T


# ----------------------------------------------------------------------------
# FP6g ([AE] App. B.2): E2M3 elements under the NVFP4 scaling hierarchy
# ----------------------------------------------------------------------------

def e2m3_value(code):
    """Value of a 6-bit E2M3 code ``s e1 e0 m2 m1 m0`` ([AE] App. B.2, Table 6:
    bias 1; exponent field 0 is subnormal, m/8; otherwise 2^(e-1)(1 + m/8))."""
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 5) & 1
    e = (code >> 3) & 3
    m = code & 7
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, e - 1))
    return np.where(s == 1, -mag, mag).astype(np.float64)


_E2M3_GRID = e2m3_value(np.arange(32))     # 0 .. 7.5, increasing


def e2m3_encode(v):
    """Nearest E2M3 value, ties to even (the even code), saturating at 7.5;
    canonical +0."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 7.5)
    hi = np.clip(np.searchsorted(_E2M3_GRID, mag, side="left"), 0, 31)
    lo = np.clip(hi - 1, 0, 31)
    dlo = np.abs(mag - _E2M3_GRID[lo])
    dhi = np.abs(_E2M3_GRID[hi] - mag)
    idx = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    sign = (v < 0) & (idx != 0)
    return (idx | (sign.astype(np.int64) << 5)).astype(np.uint8)


def fp6g_quantize(x, tensor_amax=None):
    """FP6g ([AE] App. B.2): Eqs. 2-3 with the E2M3 maximum 7.5 in place of 6:
        T = amax(X) / (7.5 * 448);  B_j = Q_E4M3(amax(X_j) / (7.5 T));
        q_i = Q_E2M3(x_i / (T B_j))
    in fp32 in that order (``sevhT = 7.5*T``; ``b = a/sevhT``; ``s = T*B``;
    ``v = x/s``), as ``nvfp4_quantize`` reads Eqs. 2-3. Returns dict(q [rows, K]
    6-bit codes, scales, T, codes = the packed bytes, rows, k)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 16")
    G = K // GROUP
    amax = np.float32(np.max(np.abs(x)) if tensor_amax is None else tensor_amax)
    T = amax / np.float32(7.5 * 448)
    sev = np.float32(7.5) * T
    a = np.max(np.abs(x.reshape(rows, G, GROUP)), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        b = (a / sev) if sev > 0 else np.zeros_like(a)
    B = R.e4m3_encode(b)
    s = (T * R.e4m3_value(B).astype(np.float32)).astype(np.float32)
    s_el = np.repeat(s, GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s_el != 0, x / np.where(s_el != 0, s_el, np.float32(1)), np.float32(0)).astype(np.float32)
    q = e2m3_encode(v)
    return dict(q=q, scales=B, T=np.float32(T), codes=pack_fp6(q), rows=rows, k=K, v=v)


def pack_fp6(q):
    """Four 6-bit codes in three bytes: code i of a quad at bits [6i+5:6i] of a
    little-endian 24-bit word. [rows, K] -> [rows, 3K/4]."""
    q = np.asarray(q, dtype=np.int64).reshape(q.shape[0], -1, 4)
    w = q[..., 0] | (q[..., 1] << 6) | (q[..., 2] << 12) | (q[..., 3] << 18)
    return np.stack([w & 0xFF, (w >> 8) & 0xFF, w >> 16], axis=-1).reshape(q.shape[0], -1).astype(np.uint8)


def unpack_fp6(b, K):
    b = np.asarray(b, dtype=np.int64).reshape(b.shape[0], -1, 3)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    return np.stack([(w >> (6 * i)) & 63 for i in range(4)], axis=-1).reshape(b.shape[0], K).astype(np.uint8)


def decode_fp6g(pk):
    """T B q in fp64 from the packed codes."""
    q = e2m3_value(unpack_fp6(pk["codes"], pk["k"]))
    return float(pk["T"]) * np.repeat(R.e4m3_value(pk["scales"]), GROUP, axis=1) * q


def linear_fp6g(wpk, xpk):
    """The FP6g comparator's W6A6 product: X_hat . W_hat^T in fp64."""
    return decode_fp6g(xpk) @ decode_fp6g(wpk).T
