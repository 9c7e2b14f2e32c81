"""Pins of the oracle against the worked examples the paper prints (CPU only)."""

import math

import numpy as np

import oracle as O
from conftest import read_golden


def _table7():
    rows = read_golden("table7_group.txt")
    xs = np.array([float(r[0]) for r in rows], np.float32)
    return rows, xs


def test_table7_base_codes_scale_mask_and_offsets():
    rows, xs = _table7()
    # x = s * (x/s) with s = 0.25 (a power of two, so x/s is recovered exactly)
    x = (xs * np.float32(0.25)).reshape(1, 16)
    base = O.nvfp4_quantize(x)
    assert int(base.scales[0, 0]) == 0x7E                 # B = 448
    assert float(base.s[0, 0]) == 0.25                     # s = T * B = 0.25 exactly
    assert base.v.ravel().tolist() == xs.tolist()
    for i, r in enumerate(rows):
        assert int(base.codes[0, i]) == int(r[2], 2), i
        assert O.e2m1_value(base.codes[0, i]) == float(r[1]), i
    bits, d = O.activation_refinement(base, None, 0.003)
    assert int(bits[0, 0]) == 0b0110                       # SG1 and SG2 refined
    for i, r in enumerate(rows):
        refined = r[3] == "1"
        assert (i // 4 in (1, 2)) == refined
        if refined:
            assert (int(d[0, i]) & 3) == int(r[4], 2), i
            assert O.e2m1_value(base.codes[0, i]) + int(d[0, i]) / 8.0 == float(r[5]), i
        else:
            assert int(d[0, i]) == 0


def test_table7_packed_activation():
    rows, xs = _table7()
    pk = O.quantize_activation((xs * np.float32(0.25)).reshape(1, 16), refine=True)
    assert pk["mask"].tolist() == [[0x06]]
    # SG1 offsets +1 +1 +1 -1 ; SG2 offsets -2 -1 +1 0 (element k in bits 2k+1:2k)
    assert pk["offsets"][0].tolist() == [0x00, 0b11010101, 0b00011110, 0x00]
    xhat = O.decode_activation(pk, 6).ravel()
    refined = [float(r[5]) for r in rows if r[3] == "1"]
    # decoded values are T * B * (q + delta) with the exact product T * B
    # (which the fp32 rounding used for the division turns into 0.25)
    tb = float(pk["T"]) * 448.0
    assert (xhat[4:12] / tb).tolist() == refined
    assert abs(tb - 0.25) < 1e-7


def test_fig23_packed_bytes():
    # masks 0110 (group 0) and 1000 (group 1) share one byte, printed MSB first
    assert int(O.pack_nibbles(np.array([0b0110, 0b1000]))[0]) == int("10000110", 2)
    # d bytes are printed in element order: 01 01 01 11 and 10 11 01 00
    for printed, d in (("01 01 01 11", [1, 1, 1, -1]), ("10 11 01 00", [-2, -1, 1, 0])):
        byte = int(O.pack_offsets_byte(np.array(d)))
        assert " ".join(format((byte >> (2 * k)) & 3, "02b") for k in range(4)) == printed


def test_fig5_nmse_and_decision():
    g = read_golden("fig5_subgroups.txt")
    sg0 = np.array([float(r[1]) for r in g if r[0] == "SG0"])
    sg1 = np.array([float(r[1]) for r in g if r[0] == "SG1"])
    q0 = np.array([float(r[2]) for r in g if r[0] == "SG0"])
    q1 = np.array([float(r[2]) for r in g if r[0] == "SG1"])
    ref1 = np.array([float(r[4]) for r in g if r[0] == "SG1"])
    printed = {r[1]: float(r[2]) for r in g if r[0] == "NMSE"}

    def nmse(x, xh):
        return float(((x - xh) ** 2).sum() / (x ** 2).sum())

    def two_sig(v):
        return float(f"{v:.1e}")

    assert two_sig(nmse(sg0, q0)) == printed["SG0"]
    assert two_sig(nmse(sg1, q1)) == printed["SG1"]
    assert two_sig(nmse(sg1, ref1)) == printed["SG1_refined"]

    # the oracle on the same normalized values (scale 1): codes, decision, offsets
    v = np.concatenate([sg0, sg1, np.zeros(8)]).astype(np.float32).reshape(1, 16)
    codes = O.e2m1_encode(v)
    assert O.e2m1_value(codes[0, :8]).tolist() == np.concatenate([q0, q1]).tolist()
    base = O.NVFP4(codes=codes, scales=np.array([[0x38]], np.uint8), T=np.float32(1),
                   v=v, s=np.array([[1.0]], np.float32))
    bits, d = O.activation_refinement(base, None, 0.003)
    assert int(bits[0, 0]) == 0b0010
    assert (O.e2m1_value(codes[0, 4:8]) + d[0, 4:8] / 8.0).tolist() == ref1.tolist()
    # excluding SG1 through the weight mask leaves it unrefined
    bits_ex, d_ex = O.activation_refinement(base, np.array([0b0010]), 0.003)
    assert int(bits_ex[0, 0]) == 0 and not d_ex.any()


def _fig26():
    return {r[0]: [float(v) for v in r[1:]] for r in read_golden("fig26_extended_k.txt")}


def _packed_unit_group(vals, d, mask_bits, positions):
    """One 16-element group with T*B = 1 holding ``vals`` at ``positions``."""
    q = np.zeros(16)
    q[positions] = vals
    codes = O.e2m1_encode(q).reshape(1, 16)
    dd = np.zeros(16, np.int64)
    dd[positions] = d
    return codes, dd


def test_fig26_extended_k_example():
    g = _fig26()
    pos = [0, 4, 8, 12]       # one element per subgroup so that masks are disjoint
    # W refines SG0 (element 0: +1/8), A refines SG2 (element 2 of the vector: -1/8)
    wc, wd = _packed_unit_group(g["W_base"], [1, 0, 0, 0], 0b0001, pos)
    ac, ad = _packed_unit_group(g["A_base"], [0, 0, -1, 0], 0b0100, pos)
    wpk = dict(codes=O.pack_nibbles(wc), scales=np.array([[0x38]], np.uint8), T=np.float32(1),
               rows=1, k=16, mask=O.pack_nibbles(np.array([0b0001])),
               offsets=O.pack_offsets_byte(wd.reshape(1, 4, 4))[:, [0]], n_refined=1)
    apk = dict(codes=O.pack_nibbles(ac), scales=np.array([[0x38]], np.uint8), T=np.float32(1),
               rows=1, k=16, mask=O.pack_nibbles(np.array([[0b0100]])),
               offsets=O.pack_offsets_byte(ad.reshape(1, 4, 4)))
    assert O.decode_weight(wpk, 6)[0, pos].tolist() == g["W_refined"]
    assert O.decode_activation(apk, 6)[0, pos].tolist() == g["A_refined"]
    assert O.linear(wpk, apk, 6)[0, 0] == g["RESULT_refined"][0]
    assert O.linear(wpk, apk, 4)[0, 0] == g["RESULT_base"][0]
    # Figure 25 construction of the extended operands, scale s_W / 4
    wq = np.array(g["W_base"])
    aq = np.array(g["A_base"])
    dw = np.array([1, 0, 0, 0]) / 8.0
    da = np.array([0, 0, -1, 0]) / 8.0
    mw = dw != 0
    ma = da != 0
    w_qr = np.where(mw, 4 * dw, np.where(ma, wq, 0.0))
    a_qr = np.where(mw, aq, np.where(ma, 4 * da, 0.0))
    assert w_qr.tolist() == g["W_qr"] and a_qr.tolist() == g["A_qr"]
    assert 0.25 * float(w_qr @ a_qr) == g["RESULT_refinement"][0]


def test_fig24_sum_of_gemms():
    g = _fig26()
    w = np.array(g["FIG24_W1"] + g["FIG24_W2"])
    a = np.array(g["FIG24_A1"] + g["FIG24_A2"])
    assert float(w @ a) == g["FIG24_Y1"][0]
    assert float(np.array(g["FIG24_W1"]) @ np.array(g["FIG24_A1"])
                 + np.array(g["FIG24_W2"]) @ np.array(g["FIG24_A2"])) == g["FIG24_Y1"][0]


def test_storage_bits_per_weight():
    # §5.1: 4 + 0.5 + 2 rho bits per weight (4.9 at rho = 0.2); masks are shared
    rng = np.random.default_rng(5)
    K = 4096
    w = (0.02 * rng.standard_normal((8, K))).astype(np.float32)
    mask, R = O.select_weight_mask(w, 0.2)
    assert R == math.floor(0.2 * K / 4) == 204
    pk = O.quantize_weight(w, O.pack_nibbles(mask))
    per_row = pk["codes"].shape[1] + pk["scales"].shape[1] + pk["offsets"].shape[1]
    bits = 8.0 * per_row / K
    assert abs(bits - (4.5 + 2 * 0.2)) < 0.005
    assert round(bits, 1) == 4.9
