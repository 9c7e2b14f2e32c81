"""GPU parity of the refinement-aware GPTQ calibration (autofp_gptq_quantize,
[AE] App. E, Algorithm 1, Eq. 7) against oracle/gptq_ref.py.

  - bit for bit (codes, scales, T, mask, offsets) on weights of 7 to 300
    rows and 48 to 2048 columns, with U and the Hessian diagonal from the
    oracle's factor of a seeded correlated calibration set: the working
    weights, the error solve and the propagation are fp64 operations in the
    order the oracle writes them, and every decision (codes, offsets, masks)
    is taken from the same values;
  - the identity Hessian gives autofp_quantize's AutoFP6 weight;
  - at the Llama-3-8B Wo shape (4096 x 4096, 2048 calibration tokens), the
    properties that hold at any size: the budget and at most two refined
    subgroups per group; group 0 (encoded from the original weights) equal
    to the oracle's encode on sampled rows; a lower Hessian-weighted error
    than encoding each weight alone with the same mask on sampled rows.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from oracle import gptq_ref as P
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def factor(k, tokens, seed):
    x = S.calibration(tokens, k, seed=seed, tensor_id=2).numpy()
    hd = P.dampen(P.hessian(x))
    return hd, P.inverse_factor(hd)


def run_gpu(w, u, h):
    return A.gptq_quantize(torch.from_numpy(w).to(DEV), torch.from_numpy(np.ascontiguousarray(u)).to(DEV),
                           torch.from_numpy(np.ascontiguousarray(h)).to(DEV))


def same(gpu, ref):
    h = gpu.to_host()
    assert np.float32(h["T"]) == np.float32(ref["T"])
    for key in ("codes", "scales", "mask", "offsets"):
        a, b = np.asarray(h[key]), np.asarray(ref[key])
        assert a.shape == b.shape, (key, a.shape, b.shape)
        bad = np.argwhere(a != b)
        assert bad.size == 0, (key, bad[:5].tolist())


@pytest.mark.parametrize("n,k,seed", [(7, 48, 0), (32, 128, 1), (64, 256, 2), (300, 512, 3), (100, 1024, 4),
                                      (128, 2048, 5)])
def test_gptq_bit_exact(n, k, seed):
    say(f"case: GPTQ {n}x{k}")
    w = S.weights(n, k, seed=seed, tensor_id=1).numpy()
    hd, u = factor(k, 4 * k, seed)
    out = run_gpu(w, u, np.diag(hd).copy())
    ref = P.gptq_quantize(w, u, np.diag(hd))
    assert out.n_refined == ref["n_refined"]
    same(out, ref)


def test_gptq_identity_hessian_is_the_encoder():
    n, k = 64, 512
    say("case: GPTQ with U = I")
    w = S.weights(n, k, seed=9, tensor_id=1)
    out = run_gpu(w.numpy(), np.eye(k), np.ones(k))
    plain = A.quantize_weight(w.to(DEV))
    for key in ("codes", "scales", "tensor_scale", "mask", "offsets"):
        assert torch.equal(getattr(out, key), getattr(plain, key)), key


def test_gptq_full_size_properties():
    n, k, tokens = 4096, 4096, 2048
    say(f"case: GPTQ {n}x{k}, {tokens} calibration tokens")
    w = S.weights(n, k, seed=11, tensor_id=1).numpy()
    hd, u = factor(k, tokens, 11)
    out = run_gpu(w, u, np.diag(hd).copy())
    h = out.to_host()
    bits = O.unpack_nibbles(h["mask"], k // 16)
    pop = np.array([bin(int(b)).count("1") for b in bits])
    assert pop.sum() == int(np.floor(0.2 * k / 4)) == out.n_refined and pop.max() <= 2
    rows = np.random.default_rng(11).choice(n, 256, replace=False)
    q0, b0, d0, _, _ = P.encode_group(w[rows, :16].astype(np.float64), np.abs(w).max())
    assert np.array_equal(O.unpack_nibbles(h["codes"][rows], k)[:, :16], q0)
    assert np.array_equal(h["scales"][rows, 0], b0)
    what = O.decode_weight(dict(h, rows=n, k=k), 6)[rows]
    rtn = O.decode_weight(O.quantize_weight(w, h["mask"]), 6)[rows]
    err = lambda d: float(np.einsum("nk,kl,nl->", d, hd, d))
    e_gptq, e_rtn = err(w[rows] - what), err(w[rows] - rtn)
    say(f"Hessian-weighted error on 256 rows: GPTQ {e_gptq:.4g}, plain encode {e_rtn:.4g}")
    assert e_gptq < 0.95 * e_rtn
