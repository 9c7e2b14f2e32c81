"""GPU parity of the batched decode GEMV (17-64 tokens per slice) and of
autofp_gemv_rows, the GEMV whose rows (tokens) run at their own precision
levels ([AE] §4.2, mixed-precision batches), against the fp64 oracle.

Tolerance as in test_gpu_linear: |y - y_ref| <= 1e-3 * max(|y_ref|,
0.01 * rms(row of y_ref)). A row at level l must match the oracle's product
at level l: W2A4 (AutoFP2 weight digits, NVFP4 activation), W4A4, or W6A6
(both operands refined; the activation with its own mask M_A)."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True)) + 1e-300
    err = np.abs(y - ref) / np.maximum(np.abs(ref), 0.01 * rms)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= RTOL, (err.max(), worst, y[worst], ref[worst])
    return float(err.max())


def packs(n, b, k, seed, rows=None):
    """GPU and oracle packings of a weight [n, k] and activations [b, k];
    ``rows`` restricts the oracle weight to those rows (full-size cases)."""
    w = S.weights(n, k, seed=seed, tensor_id=1, device=DEV)
    x = S.activations(b, k, seed=seed, tensor_id=2, device=DEV)
    wp = A.quantize_weight(w, refine=True)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
    xp4 = A.quantize_activation(x)
    wn = w.cpu().numpy()
    xn = x.float().cpu().numpy()
    bits, _ = O.select_weight_mask(wn, 0.2)
    sel = slice(None) if rows is None else rows
    wq = O.quantize_weight(wn[sel], O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    xq4 = O.quantize_activation(xn)
    xq6 = O.quantize_activation(xn, refine=True, exclude_mask=wq["mask"])
    return wp, xp4, xp6, wq, xq4, xq6


@pytest.mark.parametrize("n,b,k", [(200, 17, 256), (64, 33, 512), (300, 64, 1024), (130, 64, 4096),
                                   (1000, 48, 384), (257, 100, 4096), (70, 32, 128), (50, 20, 192),
                                   (70, 12, 4224), (130, 16, 4352), (6150, 9, 256), (48, 24, 65536)])
@pytest.mark.parametrize("level", [2, 4, 6])
def test_batched_gemv_shapes(n, b, k, level):
    """Ragged row tiles (n not a multiple of 64), 9-100 tokens (16-token tiles
    1, 2 and 4, two 64-token slices; 9-16 tokens on weights with K above 4096
    or 6144+ rows), K of 1 to 512 steps of 128, K split over blocks (small n,
    long K), and K % 128 != 0 (the other batched routes). Each block forms
    its slice of the weight mask's prefix itself (at K = 65536, the largest
    K whose masks are selected, two mask dwords per thread)."""
    say(f"case: batched GEMV n={n} b={b} k={k} level {level}")
    wp, xp4, xp6, wq, xq4, xq6 = packs(n, b, k, seed=n + b + k)
    y = A.gemv(wp, xp6 if level == 6 else xp4, bits=level).cpu().numpy()
    check_close(y, O.linear(wq, xq6 if level == 6 else xq4, level))
    # the device-side level gives the same bits
    lv = torch.tensor([level], dtype=torch.int32, device=DEV)
    yd = A.gemv(wp, xp6, bits=4, bits_dev=lv).cpu().numpy()
    if level == 6:
        assert np.array_equal(y, yd)
    else:
        check_close(yd, O.linear(wq, xq4, level))


def oracle_rows(wq, xq4, xq6, levels):
    """Row t of the oracle product at level levels[t]."""
    out = {}
    for lv in (2, 4, 6):
        out[lv] = O.linear(wq, xq6 if lv == 6 else xq4, lv)
    return np.stack([out[int(l)][t] for t, l in enumerate(levels)])


@pytest.mark.parametrize("n,b,k", [(300, 40, 1024), (130, 3, 512), (64, 70, 4096), (1000, 64, 256),
                                   (40, 20, 65536)])
def test_gemv_rows_mixed_levels(n, b, k):
    """Tokens at levels drawn from {2, 4, 6}: each output row equals the
    oracle's product at that row's level."""
    say(f"case: per-row levels n={n} b={b} k={k}")
    wp, xp4, xp6, wq, xq4, xq6 = packs(n, b, k, seed=7 * n + b)
    levels = np.random.default_rng(n + b).choice([2, 4, 6], size=b).astype(np.int32)
    lv = torch.from_numpy(levels).to(DEV)
    y = A.gemv_rows(wp, xp6, lv).cpu().numpy()
    e = check_close(y, oracle_rows(wq, xq4, xq6, levels))
    say(f"levels {np.bincount(levels, minlength=7)[[2, 4, 6]].tolist()}: max rel err {e:.2e}")


def test_gemv_rows_uniform_equals_gemv():
    """All rows at one level: the same bits as autofp_gemv at that level on the
    batched path (40 tokens), and bf16 output = RNE of the fp32 result."""
    n, b, k = 520, 40, 2048
    say("case: per-row levels, all equal")
    wp, xp4, xp6, wq, xq4, xq6 = packs(n, b, k, seed=5)
    for level in (2, 4, 6):
        lv = torch.full((b,), level, dtype=torch.int32, device=DEV)
        y_rows = A.gemv_rows(wp, xp6, lv)
        y_one = A.gemv(wp, xp6 if level == 6 else xp4, bits=level)
        assert torch.equal(y_rows, y_one), level
        yb = A.gemv_rows(wp, xp6, lv, out_dtype=torch.bfloat16)
        assert torch.equal(yb, y_rows.to(torch.bfloat16)), level


def test_gemv_rows_full_size_sampled():
    """Llama-3-8B-shaped Wo (4096 x 4096, K split over blocks) and the fused
    Wgate|Wup (28672 x 4096) at 64 tokens of mixed levels: every output of 64
    sampled weight rows (the first and last among them)."""
    for n, k, seed in ((4096, 4096, 21), (28672, 4096, 22)):
        say(f"case: per-row levels full size {n}x{k} batch 64")
        rows = np.concatenate([[0, n - 1], np.random.default_rng(seed).choice(np.arange(1, n - 1), 62, replace=False)])
        wp, xp4, xp6, wq, xq4, xq6 = packs(n, 64, k, seed=seed, rows=rows)
        levels = np.random.default_rng(seed).choice([2, 4, 6], size=64).astype(np.int32)
        y = A.gemv_rows(wp, xp6, torch.from_numpy(levels).to(DEV)).cpu().numpy()
        e = check_close(y[:, rows], oracle_rows(wq, xq4, xq6, levels))
        say(f"max rel err {e:.2e}")
