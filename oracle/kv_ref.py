"""Plain CPU reference of decode attention over an AutoFP-encoded KV cache.

TEST INFRASTRUCTURE (see the package docstring): only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

Paper: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
Exponent-Mantissa Refinement" (arXiv 2611.10165v1), cited as [AE].

What the paper fixes ([AE] §4.1, last paragraph; §5.1 hyperparameters; §3.1):
  * attention reads K and V in the same AutoFP construction as the linear
    layers: an NVFP4 base (E2M1 values, E4M3 scale per 16 elements, one FP32
    tensor scale) and, for refined tokens, signed offsets d with delta = d/8;
  * the offsets of a refined token are stored as 4*delta = d/2, which E2M1
    represents exactly ({-1, -0.5, 0, +0.5}); the factor 4 goes into the scale;
  * two page types of equal byte size: a base page holds T = 64 tokens, a
    refinement page T/2 = 32 refined tokens (base values plus offsets);
  * the 2-bit level is for weights only, so a layer at level 2 reads its KV
    cache at 4 bits (W2A4KV4).

Readings taken here (the paper leaves them open):
  * K1 groups run along the head dimension: every (token, KV head) vector is
    one row of head_dim elements, 16 per E4M3 scale.
  * K2 one FP32 tensor scale for the K cache and one for the V cache of a
    layer, T = amax / 2688 over the tokens of the call that sets it (the
    prompt); later tokens reuse it (values beyond 6 * 448 * T saturate).
  * K3 a refined token carries an offset for every subgroup, d = argmin over
    {-2, -1, 0, +1} of |x/(TB) - q - d/8| with ties to the smaller |d| (the
    same rule as the linear layers; dense storage makes a subgroup mask
    pointless for a token that already pays for a full offset vector).
  * K4 at level 6, tokens of refinement pages decode to T*B*(q + d/8) and
    tokens of base pages to T*B*q; at levels 2 and 4 every token decodes to
    T*B*q (the offsets are not read).
  * K5 the query is not quantized (the paper runs attention on a 16-bit-query
    FP8-KV kernel); scores s_j = sm_scale * q . k_hat_j, probabilities
    softmax(s) over the context, output sum_j p_j v_hat_j; query head h reads
    KV head h // (H_q / H_kv) (grouped-query attention).
"""

from __future__ import annotations

import numpy as np

from .autofp_ref import (GROUP, e2m1_encode, e2m1_value, e4m3_value, nvfp4_quantize,
                         offset_select)

__all__ = ["KV_PAGE_TOKENS", "kv_quantize", "kv_offset_codes", "kv_decode", "kv_attention"]

# [AE] §5.1: KV page size T = 64 tokens; a refinement page holds T/2 tokens.
KV_PAGE_TOKENS = 64


def kv_quantize(x, refine, tensor_amax=None):
    """Encode KV vectors x [n, head_dim] (fp32; one row per (token, KV head)).

    NVFP4 base per row ([AE] App. B.1, Eqs. 2-3) with one tensor scale over
    all rows (reading K2; ``tensor_amax`` overrides amax(x) when the scale was
    set by an earlier call). ``refine`` [n] bool marks the rows stored in
    refinement pages; they get d for every element (reading K3, [AE] §3.2).

    Returns dict(q [n, D] E2M1 codes, scales [n, D/16] E4M3 codes, T fp32,
    d [n, D] int8 (0 on rows not refined), refine [n] bool).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    base = nvfp4_quantize(x, tensor_amax)
    refine = np.broadcast_to(np.asarray(refine, dtype=bool), (x.shape[0],)).copy()
    r = base.v.astype(np.float64) - e2m1_value(base.codes)
    d = offset_select(r).astype(np.int8)
    d = np.where(refine[:, None], d, 0).astype(np.int8)
    return dict(q=base.codes.astype(np.uint8), scales=base.scales.astype(np.uint8),
                T=np.float32(base.T), d=d, refine=refine)


def kv_offset_codes(d):
    """E2M1 codes of 4*delta = d/2 for offsets d in {-2, -1, 0, +1} ([AE] §4.1:
    the scaled offset is representable in E2M1)."""
    d = np.asarray(d, dtype=np.int64)
    if np.any((d < -2) | (d > 1)):
        raise ValueError("offsets must lie in {-2, -1, 0, +1}")
    return e2m1_encode(d / 2.0)


def kv_decode(kv, level):
    """Decoded vectors [n, D] in fp64 at execution level ``level`` (reading K4):
    T*B*(q + d/8) for refined rows at level 6, T*B*q otherwise."""
    if level not in (2, 4, 6):
        raise ValueError("level must be 2, 4 or 6")
    q = e2m1_value(kv["q"])
    if level == 6:
        q = q + np.where(kv["refine"][:, None], kv["d"].astype(np.float64) / 8.0, 0.0)
    s = float(kv["T"]) * np.repeat(e4m3_value(kv["scales"]), GROUP, axis=1)
    return s * q


def kv_attention(q, k_hat, v_hat, sm_scale):
    """Decode attention of one sequence (reading K5), fp64.

    q [H_q, D]; k_hat, v_hat [H_kv, L, D] decoded K and V; returns [H_q, D]:
    out[h] = sum_j softmax_j(sm_scale * q[h] . k_hat[g, j]) * v_hat[g, j] with
    g = h // (H_q / H_kv). The softmax subtracts the row maximum first.
    """
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    hq, hkv = q.shape[0], k_hat.shape[0]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    grp = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    for h in range(hq):
        g = h // grp
        s = float(sm_scale) * (k_hat[g] @ q[h])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ v_hat[g]
    return out
