"""Pins of the KV-cache oracle (CPU only).

Each test fixes a part of oracle/kv_ref.py with something other than the
oracle itself: the paper's worked example ([AE] App. B.5, Table 7), the
statement that 4*delta is an E2M1 value ([AE] §4.1), brute force in exact
arithmetic, and closed forms of softmax attention (two tokens: the logistic
function; equal scores: the mean; duplicated context; a constant shift of V).
"""

import math
from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O
from conftest import read_golden
from fp_exact import round_f32

RNG = np.random.default_rng(1234)


def test_offset_codes_are_e2m1_of_four_delta():
    # [AE] §4.1: 4*delta in {-1, -0.5, 0, +0.5} is representable in E2M1
    for d, code in ((-2, 0b1010), (-1, 0b1001), (0, 0b0000), (1, 0b0001)):
        c = int(O.kv_offset_codes(np.array([d]))[0])
        assert c == code, (d, c)
        assert float(O.e2m1_value(c)) == d / 2.0
    with pytest.raises(ValueError):
        O.kv_offset_codes(np.array([2]))


def test_refined_token_reproduces_table7():
    rows = read_golden("table7_group.txt")
    xs = np.array([float(r[0]) for r in rows], np.float32)
    x = (xs * np.float32(0.25)).reshape(1, 16)
    kv = O.kv_quantize(x, refine=[True])
    assert int(kv["scales"][0, 0]) == 0x7E
    # the printed refined elements: same d code and q + delta
    for i, r in enumerate(rows):
        assert int(kv["q"][0, i]) == int(r[2], 2), i
        if r[3] == "1":
            assert (int(kv["d"][0, i]) & 3) == int(r[4], 2), i
    xhat = O.kv_decode(kv, 6).ravel()
    tb = float(kv["T"]) * 448.0
    got = (xhat / tb)[4:12].tolist()
    assert got == [float(r[5]) for r in rows if r[3] == "1"]
    # every element (also SG0 and SG3, which Table 7 leaves unrefined) gets the
    # exact argmin over the four candidates, ties to the smaller |d|
    for i in range(16):
        v = F(float(xs[i]))
        q = F(float(O.e2m1_value(kv["q"][0, i])))
        best = min((0, 1, -1, -2), key=lambda d: (abs(v - q - F(d, 8)), abs(d)))
        assert int(kv["d"][0, i]) == best, i


def test_base_token_is_plain_nvfp4_and_level_rules():
    x = RNG.standard_normal((6, 128)).astype(np.float32)
    refine = np.array([False, True, False, True, True, False])
    kv = O.kv_quantize(x, refine)
    # base codes and scales do not depend on refinement: the activation
    # quantizer (pinned by the Table 7 and brute-force tests) gives the same
    act = O.quantize_activation(x)
    assert np.array_equal(O.pack_nibbles(kv["q"]), act["codes"])
    assert np.array_equal(kv["scales"], act["scales"])
    assert np.float32(kv["T"]) == np.float32(act["T"])
    assert not kv["d"][~refine].any()
    # level 4 (and 2: W2A4KV4) ignores offsets; level 6 adds them on refined rows
    b4, b2, b6 = O.kv_decode(kv, 4), O.kv_decode(kv, 2), O.kv_decode(kv, 6)
    assert np.array_equal(b4, b2)
    assert np.array_equal(b6[~refine], b4[~refine])
    s = float(kv["T"]) * np.repeat(O.e4m3_value(kv["scales"]), 16, axis=1)
    assert np.array_equal(b6[refine], (s * (O.e2m1_value(kv["q"]) + kv["d"] / 8.0))[refine])
    # refinement never increases the error of an element (argmin includes d = 0)
    err4 = np.abs(b4 - x)[refine]
    err6 = np.abs(b6 - x)[refine]
    assert np.all(err6 <= err4 + 1e-12)
    assert err6.sum() < err4.sum()


def test_given_tensor_scale_is_used():
    x = RNG.standard_normal((3, 32)).astype(np.float32)
    kv = O.kv_quantize(x, [False] * 3, tensor_amax=np.float32(100.0))
    assert np.float32(kv["T"]) == np.float32(100.0) / np.float32(2688.0)
    # a group of amax a gets the E4M3 code of round_f32(a / round_f32(6 T))
    T = F(float(kv["T"]))
    sixt = round_f32(6 * T)
    a = F(float(np.max(np.abs(x[0, :16]))))
    b = float(round_f32(a / sixt))
    assert int(kv["scales"][0, 0]) == int(O.e4m3_encode(np.array([b]))[0])


def _two_token_closed_form(q, k, v, sc):
    s1, s2 = sc * float(q @ k[0]), sc * float(q @ k[1])
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))           # logistic
    return w1 * v[0] + (1.0 - w1) * v[1]


def test_attention_two_tokens_is_logistic_mix():
    q = RNG.standard_normal((1, 16))
    k = RNG.standard_normal((1, 2, 16))
    v = RNG.standard_normal((1, 2, 16))
    out = O.kv_attention(q, k, v, 0.25)
    ref = _two_token_closed_form(q[0], k[0], v[0], 0.25)
    assert np.allclose(out[0], ref, rtol=1e-13, atol=1e-15)


def test_attention_equal_scores_give_mean_and_dominant_token_wins():
    L, D = 37, 32
    v = RNG.standard_normal((1, L, D))
    k = RNG.standard_normal((1, L, D))
    out = O.kv_attention(np.zeros((1, D)), k, v, 1.0)
    assert np.allclose(out[0], v[0].mean(axis=0), rtol=1e-13, atol=1e-15)
    # one score 80 above the rest: the output is that token's value
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k2 = np.zeros((1, L, D))
    k2[0, 11, 0] = 80.0
    out = O.kv_attention(q, k2, v, 1.0)
    assert np.allclose(out[0], v[0, 11], rtol=1e-30, atol=1e-30 + 1e-33 * L * np.abs(v).max())
    assert np.max(np.abs(out[0] - v[0, 11])) <= L * math.exp(-80.0) * np.abs(v).max() * 2


def test_attention_invariances_and_head_mapping():
    hq, hkv, L, D = 8, 2, 23, 16
    q = RNG.standard_normal((hq, D))
    k = RNG.standard_normal((hkv, L, D))
    v = RNG.standard_normal((hkv, L, D))
    out = O.kv_attention(q, k, v, 0.3)
    # permuting the context changes nothing
    perm = RNG.permutation(L)
    assert np.allclose(O.kv_attention(q, k[:, perm], v[:, perm], 0.3), out, rtol=1e-12, atol=1e-14)
    # every token twice: the same weights after normalization
    kk, vv = np.concatenate([k, k], axis=1), np.concatenate([v, v], axis=1)
    assert np.allclose(O.kv_attention(q, kk, vv, 0.3), out, rtol=1e-12, atol=1e-14)
    # KV head 1 := KV head 0 with V shifted by c: heads 4..7 (group 1) equal
    # heads 0..3 plus c, since the weights sum to one
    c = RNG.standard_normal(D)
    k1 = np.stack([k[0], k[0]])
    v1 = np.stack([v[0], v[0] + c])
    q1 = np.concatenate([q[:4], q[:4]])
    o1 = O.kv_attention(q1, k1, v1, 0.3)
    assert np.allclose(o1[4:], o1[:4] + c, rtol=1e-12, atol=1e-13)
    # a single-token context returns that token's value for every head
    o = O.kv_attention(q, k[:, :1], v[:, :1], 0.3)
    assert np.array_equal(o, np.repeat(v[:, 0], hq // hkv, axis=0))
