"""GPU parity of the format variants ([AE] §6.5 / Fig. 14(a): the
exponent-scaled offset step; App. I / Table 10: AutoFP8, 4-bit offsets;
App. B.2: the FP6g comparator) against the oracle of oracle/formats_ref.py.

  - encode (activations with and without refinement and an exclusion mask;
    weights with their mask): codes, scales, T, masks and offsets bit for bit,
    on both encode paths (one launch / amax partials first);
  - weight-mask selection with each format's gains: the same mask bytes;
  - the linear layer at every level a format runs (AUTOFP6E 2/4/6, AUTOFP8
    2/4/6/8, FP6G 6) through autofp_gemv (1-64 tokens) and autofp_gemm
    (prefill tiles), ragged row counts, within the tolerance of
    test_gpu_linear: |y - y_ref| <= 1e-3 * max(|y_ref|, 0.01 rms(row));
  - the device-side level gives the same bits as the host level.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle.formats_ref as V
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-3
OFFSET_FORMATS = ("autofp6e", "autofp8")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same(gpu, ref, keys):
    h = gpu.to_host()
    for key in keys:
        if key == "T":
            assert np.float32(h["T"]) == np.float32(ref["T"])
            continue
        a, b = np.asarray(h[key]), np.asarray(ref[key])
        assert a.shape == b.shape, (key, a.shape, b.shape)
        bad = np.argwhere(a != b)
        assert bad.size == 0, (key, bad[:5].tolist())


def check_close(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True)) + 1e-300
    err = np.abs(y - ref) / np.maximum(np.abs(ref), 0.01 * rms)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= RTOL, (err.max(), worst, y[worst], ref[worst])
    return float(err.max())


@pytest.mark.parametrize("fmt", OFFSET_FORMATS)
@pytest.mark.parametrize("rows,k", [(1, 4096), (1, 14336), (3, 272), (64, 4096), (16, 14336)])
@pytest.mark.parametrize("refine", [False, True])
def test_encode_activation_offset_formats(fmt, rows, k, refine):
    say(f"case: encode activation {fmt} {rows}x{k} refine={refine}")
    x = S.activations(rows, k, seed=rows + k, tensor_id=1, dtype=torch.bfloat16, device=DEV)
    g = torch.Generator().manual_seed(k)
    excl = torch.randint(0, 256, ((k + 31) // 32,), generator=g, dtype=torch.uint8).to(DEV)
    ex = excl if refine else None
    pk = A.quantize_activation(x, refine=refine, exclude_mask=ex, format=fmt)
    ref = V.quantize_activation_fmt(x.float().cpu().numpy(), fmt, refine=refine,
                                    exclude_mask=None if ex is None else excl.cpu().numpy())
    same(pk, ref, ("codes", "scales", "T") + (("mask", "offsets") if refine else ()))


@pytest.mark.parametrize("rows,k", [(1, 4096), (1, 14336), (3, 272), (64, 4096), (5, 65536)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_encode_fp6g(rows, k, dtype):
    say(f"case: encode FP6g {rows}x{k} {dtype}")
    x = S.activations(rows, k, seed=3 * rows + k, tensor_id=2, dtype=dtype, device=DEV)
    pk = A.quantize_activation(x, format="fp6g")
    ref = V.fp6g_quantize(x.float().cpu().numpy())
    same(pk, ref, ("codes", "scales", "T"))
    assert pk.mask is None and pk.offsets is None


@pytest.mark.parametrize("fmt", OFFSET_FORMATS)
@pytest.mark.parametrize("n,k", [(64, 256), (300, 1024), (128, 4096)])
def test_weight_mask_and_encode(fmt, n, k):
    say(f"case: weight mask + encode {fmt} {n}x{k}")
    w = S.weights(n, k, seed=n + k, tensor_id=3, device=DEV)
    wp = A.quantize_weight(w, format=fmt)
    wn = w.cpu().numpy()
    bits, R = V.select_weight_mask_fmt(wn, fmt, 0.2)
    assert wp.n_refined == R
    assert np.array_equal(wp.mask.cpu().numpy(), O.pack_nibbles(bits))
    ref = V.quantize_weight_fmt(wn, fmt, mask=O.pack_nibbles(bits))
    same(wp, ref, ("codes", "scales", "T", "mask", "offsets"))


def test_fp6g_weight_encode():
    say("case: FP6g weight encode 300x1024")
    w = S.weights(300, 1024, seed=4, tensor_id=3, device=DEV)
    wp = A.quantize_weight(w, format="fp6g")
    same(wp, V.fp6g_quantize(w.cpu().numpy()), ("codes", "scales", "T"))


def packs(fmt, n, b, k, seed, rows=None):
    """GPU and oracle packings of W [n, k] and X [b, k] in format fmt
    (``rows`` restricts the oracle weight to those rows)."""
    w = S.weights(n, k, seed=seed, tensor_id=1, device=DEV)
    x = S.activations(b, k, seed=seed, tensor_id=2, device=DEV)
    wn, xn = w.cpu().numpy(), x.float().cpu().numpy()
    sel = slice(None) if rows is None else rows
    if fmt == "fp6g":
        wp = A.quantize_weight(w, format=fmt)
        xp = A.quantize_activation(x, format=fmt)
        wq = V.fp6g_quantize(wn[sel], tensor_amax=np.abs(wn).max())
        return wp, xp, xp, wq, None, V.fp6g_quantize(xn)
    wp = A.quantize_weight(w, format=fmt)
    xp4 = A.quantize_activation(x, format=fmt)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask, format=fmt)
    bits, _ = V.select_weight_mask_fmt(wn, fmt, 0.2)
    wq = V.quantize_weight_fmt(wn[sel], fmt, mask=O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    xq4 = V.quantize_activation_fmt(xn, fmt)
    xq6 = V.quantize_activation_fmt(xn, fmt, refine=True, exclude_mask=wq["mask"])
    return wp, xp4, xp6, wq, xq4, xq6


def levels_of(fmt):
    return {"autofp6e": (2, 4, 6), "autofp8": (2, 4, 6, 8), "fp6g": (6,)}[fmt]


def oracle_linear(fmt, wq, xq4, xq6, level):
    if fmt == "fp6g":
        return V.linear_fp6g(wq, xq6)
    return V.linear_fmt(wq, xq6 if level >= 6 else xq4, level)


@pytest.mark.parametrize("fmt", ("autofp6e", "autofp8", "fp6g"))
@pytest.mark.parametrize("n,b,k", [(300, 1, 1024), (130, 5, 512), (520, 64, 2048), (200, 40, 64),
                                   (1000, 300, 1024), (301, 2, 4160), (77, 8, 64), (64, 3, 14336),
                                   (9, 1, 256), (45, 4, 256), (33, 2, 14336), (50, 1, 16448)])
def test_linear_formats(fmt, n, b, k):
    """Every level of the format on the decode entry point (and the prefill
    one at the same shape): ragged weight rows, 1-300 tokens (1-4 on the
    vector GEMV, K from 64 (fewer items than lanes) to 16448; tokens x K up
    to 16384 with the activations decoded in the kernel, beyond it and at 3-4
    tokens from the panel)."""
    say(f"case: linear {fmt} n={n} b={b} k={k}")
    wp, xp4, xp6, wq, xq4, xq6 = packs(fmt, n, b, k, seed=n + b + k)
    for level in levels_of(fmt):
        xp = xp6 if level >= 6 else xp4
        ref = oracle_linear(fmt, wq, xq4, xq6, level)
        y = A.gemv(wp, xp, bits=level).cpu().numpy()
        e = check_close(y, ref)
        yg = A.gemm(wp, xp, bits=level).cpu().numpy()
        check_close(yg, ref)
        say(f"level {level}: max rel err {e:.2e}")


def test_linear_formats_device_level():
    """AutoFP8 and AutoFP6E with the level read on the device: the same bits
    as the host level (both run the format's GEMM tiles)."""
    for fmt in OFFSET_FORMATS:
        say(f"case: device level {fmt}")
        wp, xp4, xp6, wq, xq4, xq6 = packs(fmt, 256, 8, 1024, seed=11)
        for level in levels_of(fmt):
            if level < 6:
                continue
            lv = torch.tensor([level], dtype=torch.int32, device=DEV)
            y_host = A.gemv(wp, xp6, bits=level)
            y_dev = A.gemv(wp, xp6, bits=4, bits_dev=lv)
            assert torch.equal(y_host, y_dev), (fmt, level)


def test_linear_formats_shape_rules():
    """Levels above 4 of a variant format need k % 64 == 0; levels 2 and 4
    run on the AutoFP6 kernels at any k % 16 == 0."""
    wp, xp4, xp6, wq, xq4, xq6 = packs("autofp8", 100, 3, 272, seed=5)
    with pytest.raises(A.AutofpError):
        A.gemv(wp, xp6, bits=8)
    check_close(A.gemv(wp, xp4, bits=4).cpu().numpy(), oracle_linear("autofp8", wq, xq4, xq6, 4))


@pytest.mark.parametrize("fmt", ("autofp6e", "autofp8", "fp6g"))
@pytest.mark.parametrize("b", [1, 4])
def test_decode_formats_full_width_sampled(fmt, b):
    """The one-token decode the benchmark times (Wup 14336 x 4096) and 4
    tokens (the vector GEMV's widest case), at the format's top level: every output of 48 sampled weight
    rows (the first and last among them), fp32 and bf16 outputs."""
    n, k = 14336, 4096
    rows = np.concatenate([[0, n - 1], np.random.default_rng(8).choice(np.arange(1, n - 1), 46, replace=False)])
    say(f"case: decode {fmt} {n}x{k} at {b} tokens, sampled rows")
    wp, xp4, xp6, wq, xq4, xq6 = packs(fmt, n, b, k, seed=33, rows=rows)
    level = 8 if fmt == "autofp8" else 6
    ref = oracle_linear(fmt, wq, xq4, xq6, level)
    y = A.gemv(wp, xp6, bits=level, out_dtype=torch.float32).cpu().numpy()
    e = check_close(y[:, rows], ref)
    yb = A.gemv(wp, xp6, bits=level, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.abs(yb[:, rows] - y[:, rows]).max() <= 2.0 ** -8 * np.abs(y[:, rows]).max()
    say(f"max rel err {e:.2e}")


@pytest.mark.parametrize("fmt", ("autofp6e", "autofp8", "fp6g"))
def test_prefill_formats_full_width_sampled(fmt):
    """Llama-3-8B Wgate-shaped weight (14336 x 4096) at 512 prompt tokens:
    every output of 48 sampled weight rows (the first and last among them)."""
    n, b, k = 14336, 512, 4096
    rows = np.concatenate([[0, n - 1], np.random.default_rng(7).choice(np.arange(1, n - 1), 46, replace=False)])
    say(f"case: prefill {fmt} {n}x{k} at {b} tokens, sampled rows")
    wp, xp4, xp6, wq, xq4, xq6 = packs(fmt, n, b, k, seed=31, rows=rows)
    level = 8 if fmt == "autofp8" else 6
    y = A.gemm(wp, xp6, bits=level, out_dtype=torch.float32).cpu().numpy()
    e = check_close(y[:, rows], oracle_linear(fmt, wq, xq4, xq6, level))
    say(f"max rel err {e:.2e}")
