"""Pins of the oracle's linear layer, signals and policy (CPU only)."""

import math
from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O
from conftest import read_golden

E2M1 = [F(v) for v in {r[0]: r[1:] for r in read_golden("formats.txt")}["E2M1"]]


def _code_value(nib):
    mag = E2M1[nib & 7]
    return -mag if nib & 8 else mag


def _e4m3_exact(code):
    e, m = (code >> 3) & 15, code & 7
    return F(m, 8) * F(1, 64) if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7)


def _dec_bytes(codes, scales, T, K, deltas=None, level=4, c2=2):
    """Exact decode straight from the packed bytes (independent bit parsing)."""
    rows = codes.shape[0]
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(codes[r, k // 2])
            nib = byte & 0xF if k % 2 == 0 else byte >> 4
            s = F(float(T)) * _e4m3_exact(int(scales[r, k // 16]))
            if level == 2:
                e1, e0 = (nib >> 2) & 1, (nib >> 1) & 1
                q = 2 * (e1 & e0) + (e1 ^ e0)
                row.append(c2 * s * (-q if nib & 8 else q))
            else:
                q = _code_value(nib)
                if deltas is not None:
                    q += deltas[r][k]
                row.append(s * q)
        out.append(row)
    return out


def _dense_deltas_from_bytes(offsets, rows, K):
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(offsets[r, k // 4])
            d = (byte >> (2 * (k % 4))) & 3
            row.append(F(d - 4 if d >= 2 else d, 8))
        out.append(row)
    return out


def _weight_deltas_from_bytes(offsets, mask, rows, K):
    out = []
    for r in range(rows):
        row, col = [F(0)] * K, 0
        for j in range(K // 16):
            mb = int(mask[j // 2]) >> (4 * (j % 2))
            for sg in range(4):
                if (mb >> sg) & 1:
                    byte = int(offsets[r, col])
                    col += 1
                    for e in range(4):
                        d = (byte >> (2 * e)) & 3
                        row[16 * j + 4 * sg + e] = F(d - 4 if d >= 2 else d, 8)
        out.append(row)
    return out


@pytest.mark.parametrize("level", [2, 4, 6])
def test_linear_matches_exact_bruteforce(level):
    rng = np.random.default_rng(level)
    K = 64
    w = (0.02 * rng.standard_normal((3, K))).astype(np.float32)
    x = rng.standard_normal((2, K)).astype(np.float32)
    x[0, 5] *= 20
    mask, R = O.select_weight_mask(w, 0.25)
    wpk = O.quantize_weight(w, O.pack_nibbles(mask))
    xpk = O.quantize_activation(x, refine=(level == 6), exclude_mask=wpk["mask"])
    y = O.linear(wpk, xpk, level)
    if level == 6:
        wd = _weight_deltas_from_bytes(wpk["offsets"], wpk["mask"], 3, K)
        xd = _dense_deltas_from_bytes(xpk["offsets"], 2, K)
        W = _dec_bytes(wpk["codes"], wpk["scales"], wpk["T"], K, wd)
        X = _dec_bytes(xpk["codes"], xpk["scales"], xpk["T"], K, xd)
    else:
        W = _dec_bytes(wpk["codes"], wpk["scales"], wpk["T"], K, level=level)
        X = _dec_bytes(xpk["codes"], xpk["scales"], xpk["T"], K)
    for b in range(2):
        for n in range(3):
            exact = sum(X[b][k] * W[n][k] for k in range(K))
            assert abs(F(float(y[b, n])) - exact) <= abs(exact) * F(1, 10 ** 12) + F(1, 10 ** 30)


def test_six_bit_equals_extended_k_construction():
    """Eq. 5 / Fig. 25: base GEMM + (s_W/4)-scaled GEMM over the extended
    operands equals the product of the refined operands when masks are disjoint."""
    rng = np.random.default_rng(21)
    K = 256
    w = (0.02 * rng.standard_normal((6, K))).astype(np.float32)
    x = rng.standard_normal((4, K)).astype(np.float32)
    mask, _ = O.select_weight_mask(w, 0.2)
    wpk = O.quantize_weight(w, O.pack_nibbles(mask))
    xpk = O.quantize_activation(x, refine=True, exclude_mask=wpk["mask"])
    Wq = O.decode_weight(wpk, 4)
    Xq = O.decode_activation(xpk, 4)
    sw = float(wpk["T"]) * np.repeat(O.e4m3_value(wpk["scales"]), 16, axis=1)
    sa = float(xpk["T"]) * np.repeat(O.e4m3_value(xpk["scales"]), 16, axis=1)
    dW = (O.decode_weight(wpk, 6) - Wq) / sw          # delta_W in NVFP4 units
    dA = (O.decode_activation(xpk, 6) - Xq) / sa
    mW = np.repeat(((wpk["mask_bits"][:, None] >> np.arange(4)) & 1).reshape(-1), 4).astype(bool)
    y = O.linear(wpk, xpk, 4)
    for b in range(4):
        mA = np.repeat(((xpk["mask_bits"][b][:, None] >> np.arange(4)) & 1).reshape(-1), 4).astype(bool)
        assert not (mA & mW).any()
        for n in range(6):
            w_qr = np.where(mW, 4 * dW[n], np.where(mA, Wq[n] / sw[n], 0.0))
            a_qr = np.where(mW, Xq[b] / sa[b], np.where(mA, 4 * dA[b], 0.0))
            ext = y[b, n] + float(np.sum((sw[n] / 4) * w_qr * sa[b] * a_qr))
            assert ext == pytest.approx(O.linear(wpk, xpk, 6)[b, n], rel=1e-12, abs=1e-15)


def test_level2_levels():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((4, 64)).astype(np.float32)
    pk = O.quantize_weight(w)
    s = float(pk["T"]) * np.repeat(O.e4m3_value(pk["scales"]), 16, axis=1)
    units = O.decode_weight(pk, 2) / s
    assert set(np.unique(units).tolist()) <= {-4.0, -2.0, 0.0, 2.0, 4.0}
    q = np.abs(O.decode_weight(pk, 4) / s)
    assert (np.abs(units)[(q >= 1) & (q <= 3)] == 2).all()
    assert (np.abs(units)[q <= 0.5] == 0).all()
    assert (np.abs(units)[q >= 4] == 4).all()


def test_entropy_closed_forms():
    V = 1000
    z = np.full((1, V), -50.0)
    z[0, :10] = 3.0                           # ten equal top logits
    assert O.topk_entropy(z, 10)[0] == pytest.approx(1.0, abs=1e-15)
    z2 = np.zeros((1, V))
    z2[0, 7] = 60.0                           # one dominant logit
    assert O.topk_entropy(z2, 10)[0] < 1e-18
    # m logits at a, 10 - m at a - t: p1 = 1 / (m + (10-m) e^-t)
    for m, t in ((3, 1.0), (5, 0.25), (1, 4.0)):
        z3 = np.full((1, V), -100.0)
        z3[0, :m] = 2.0
        z3[0, m:10] = 2.0 - t
        p1 = 1.0 / (m + (10 - m) * math.exp(-t))
        p2 = p1 * math.exp(-t)
        h = -(m * p1 * math.log(p1) + (10 - m) * p2 * math.log(p2))
        assert O.topk_entropy(z3, 10)[0] == pytest.approx(h / math.log(10), rel=1e-13)
    # only the top K matter
    z4 = z3.copy()
    z4[0, 500:] = -20.0
    assert O.topk_entropy(z4, 10)[0] == O.topk_entropy(z3, 10)[0]
    # full vocabulary (k >= V): uniform -> 1
    assert O.topk_entropy(np.zeros((1, 37)), 10 ** 6)[0] == pytest.approx(1.0, abs=1e-14)


def test_update_norm_closed_forms():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((3, 4096))
    nrm = np.linalg.norm(h, axis=1)
    for a in (0.5, -0.25, 0.0):
        got = O.update_norm(h, (1 + a) * h, 1e-6)
        assert got == pytest.approx(abs(a) * nrm / (nrm + 1e-6), rel=1e-12, abs=1e-15)
    u = rng.standard_normal(4096)
    u -= (u @ h[0]) / (h[0] @ h[0]) * h[0]
    u *= 3.0 / np.linalg.norm(u)
    got = O.update_norm(h[:1], h[:1] + u, 0.0)[0]
    assert got == pytest.approx(3.0 / nrm[0], rel=1e-12)


def test_prefill_policy_spike_then_trend():
    # flat metric, spike at layer 3, then two layers below mu lower the next
    la = [1.0, 1.02, 0.98, 9.0, 0.5, 0.4, 0.45, 0.4, 5.0, 6.0, 7.0]
    bits = O.policy_prefill(la)
    # layers 0..3 (spike included) at 6; layers 4,5 below mu -> layer 6 at 4;
    # layers 6,7 below mu -> layer 8 at 2; layers 8,9 above -> layer 10 at 4
    assert bits == [6, 6, 6, 6, 6, 6, 4, 4, 2, 2, 4]
    # no spike -> all layers at 6
    assert O.policy_prefill([1.0, 1.1, 0.9, 1.05, 0.95, 1.0]) == [6] * 6


def test_decode_policy_regimes():
    st = O.PolicyState()
    for m in (0.0, 1.0, 0.0, 1.0):     # earlier steps: mu = 0.5 in metric units
        st.add(m)
    # high entropy: beta = 2 layers above raise, alpha = 4 below lower
    g = 0.5
    up = [(1.0 - 0.3 * g) / 0.7] * 2 + [0.0] * 6
    bits = O.policy_decode_step(up, g, st)
    # layers 0,1 above mu -> layer 2 at 6; layers 2..5 below -> layer 6 at 4
    assert bits == [4, 4, 6, 6, 6, 6, 4, 4]
    st2 = O.PolicyState()
    for m in (0.0, 1.0, 0.0, 1.0):
        st2.add(m)
    # low entropy: alpha = 4 layers above needed to raise; beta = 2 below lower
    g = 0.05
    hi = (1.0 - 0.3 * g) / 0.7
    bits = O.policy_decode_step([hi, hi, hi, hi, 0.0, 0.0, 0.0], g, st2)
    # layers 0..3 above -> layer 4 at 6; layers 4,5 below -> layer 6 at 4
    assert bits == [4, 4, 4, 4, 6, 6, 4]
    # alternating blips never reach a two-in-a-row trend at the default lengths
    st3 = O.PolicyState()
    for m in (0.4, 0.6):
        st3.add(m)
    blips = [1.5, 0.0] * 5
    assert O.policy_decode_step(blips, 0.05, st3) == [4] * 10
