"""GPU parity of the AutoFP decode GEMV and prefill GEMM against the fp64
oracle product of the decoded operands.

Tolerance: the products are exact and only the fp32 accumulation rounds, so
every output must satisfy |y - y_ref| <= 1e-3 * max(|y_ref|, 0.01 * rms(y_ref
row)) (relative error 1e-3, guarded near zero crossings of the output)."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import _native as N
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
    den = np.maximum(np.abs(ref), 0.01 * rms)
    err = np.abs(y - ref) / den
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= RTOL, (err.max(), worst, y[worst], ref[worst])
    return float(err.max())


def operands(n, b, k, seed, outliers=0.01, wdev=DEV):
    w = S.weights(n, k, seed=seed, tensor_id=1, device=wdev)
    x = S.activations(b, k, seed=seed, tensor_id=2, outlier_frac=outliers, device=wdev)
    return w, x


def gpu_pack(w, x):
    wp = A.quantize_weight(w, refine=True)
    xp4 = A.quantize_activation(x)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
    return wp, xp4, xp6


def oracle_pack(w, x):
    wn = w.cpu().numpy()
    xn = x.float().cpu().numpy()
    bits, _ = O.select_weight_mask(wn, 0.2)
    wq = O.quantize_weight(wn, O.pack_nibbles(bits))
    xq4 = O.quantize_activation(xn)
    xq6 = O.quantize_activation(xn, refine=True, exclude_mask=wq["mask"])
    return wq, xq4, xq6


def run(fn, wp, xp4, xp6, level, **kw):
    return fn(wp, xp6 if level == 6 else xp4, bits=level, **kw)


@pytest.mark.parametrize("level", [2, 4, 6])
@pytest.mark.parametrize("op", ["gemv", "gemm"])
def test_config1_layer(level, op):
    """16x256 bf16 activations (1% outliers x20) times a 256x256 weight."""
    say(f"case: C1 {op} level {level}")
    w = S.weights(256, 256, seed=0, tensor_id=2, heavy_frac=0.0, device=DEV)
    x = S.activations(16, 256, seed=0, tensor_id=1, device=DEV)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    y = run(getattr(A, op), wp, xp4, xp6, level)
    ref = O.linear(wq, xq6 if level == 6 else xq4, level)
    check_close(y.cpu().numpy(), ref)


SHAPES = [  # (N, B, K)
    (200, 1, 272), (200, 3, 4096 + 16), (64, 8, 512), (48, 16, 256), (130, 17, 384),
    (96, 33, 1024), (40, 64, 128), (72, 100, 160), (16, 5, 16), (50, 20, 272),
]


@pytest.mark.parametrize("n,b,k", SHAPES)
@pytest.mark.parametrize("level", [2, 4, 6])
def test_gemv_shapes(n, b, k, level):
    say(f"case: gemv N={n} B={b} K={k} level {level}")
    w, x = operands(n, b, k, seed=n * 7 + b)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    y = run(A.gemv, wp, xp4, xp6, level)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


GEMM_SHAPES = [(200, 130, 272), (384, 512, 1024), (128, 1, 64), (260, 129, 4096 + 16), (64, 300, 96),
               (1000, 300, 512), (72, 257, 192), (8200, 2000, 128), (300, 256, 64), (520, 1000, 2048),
               (64, 130, 32768), (40, 129, 32768 + 64)]


@pytest.mark.parametrize("n,m,k", GEMM_SHAPES)
@pytest.mark.parametrize("level", [2, 4, 6])
def test_gemm_shapes(n, m, k, level):
    """Ragged tiles in M and N for both GEMM kernels; 8200 x 2000 x 128 takes
    the 256 x 256 tiles (264 blocks), the other 128+ token shapes with
    K % 64 == 0 the 256 x 128 (K = 64: a single step; K = 192: an odd step
    count; K = 32768 and 32832: long K loops)."""
    say(f"case: gemm N={n} M={m} K={k} level {level}")
    w, x = operands(n, m, k, seed=n + m + k, outliers=0.005)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    y = run(A.gemm, wp, xp4, xp6, level)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))
    if level == 4:
        yb = run(A.gemm, wp, xp4, xp6, level, out_dtype=torch.bfloat16)
        assert torch.equal(yb, y.to(torch.bfloat16)), "bf16 output is not the RNE of the fp32 result"


@pytest.mark.parametrize("op,n,b", [("gemv", 96, 12), ("gemm", 96, 12), ("gemv", 200, 40), ("gemv", 8200, 40),
                                    ("gemm", 300, 200)])
def test_bf16_output_and_device_level(op, n, b):
    """bf16 outputs are the fp32 results rounded; a level read on the device
    gives the host-level result, bit for bit (40 tokens: the panel kernel,
    which reads packed activations at host levels 2 and 4 and the fp16 panel
    for a device-side level; 8200 rows: the 64-token GEMM tile)."""
    say(f"case: {op} bf16 output and device-side level N={n} B={b}")
    w, x = operands(n, b, 512, seed=4)
    wp, xp4, xp6 = gpu_pack(w, x)
    fn = getattr(A, op)
    for level in (2, 4, 6):
        y32 = fn(wp, xp6, bits=level)
        y16 = fn(wp, xp6, bits=level, out_dtype=torch.bfloat16)
        assert torch.equal(y16, y32.to(torch.bfloat16))
        dev_bits = torch.tensor([level], dtype=torch.int32, device=DEV)
        yd = fn(wp, xp6, bits=0, bits_dev=dev_bits)
        if level != 6:
            # the activation carries refinement, unused below level 6
            assert torch.equal(yd, fn(wp, xp4 if level != 6 else xp6, bits=level))
        else:
            assert torch.equal(yd, y32)


def test_gemv_equals_gemm():
    say("case: gemv vs gemm agreement")
    w, x = operands(300, 40, 1024, seed=9)
    wp, xp4, xp6 = gpu_pack(w, x)
    for level in (2, 4, 6):
        xa = xp6 if level == 6 else xp4
        a = A.gemv(wp, xa, bits=level).cpu().numpy()
        b = A.gemm(wp, xa, bits=level).cpu().numpy()
        assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max()


def test_saved_and_loaded_operands_give_identical_outputs(tmp_path):
    say("case: save/load round trip 4096x4096, 1 and 40 tokens")
    w, x = operands(4096, 40, 4096, seed=21)
    wp, xp4, xp6 = gpu_pack(w, x)
    path = tmp_path / "layer.safetensors"
    A.save_packed(path, {"w": wp, "x4": xp4, "x6": xp6})
    got = A.load_packed(path, device=DEV)
    for level in (2, 4, 6):
        xa, xb = (xp6, got["x6"]) if level == 6 else (xp4, got["x4"])
        for fn in (A.gemv, A.gemm):
            assert torch.equal(fn(wp, xa, bits=level), fn(got["w"], xb, bits=level)), (fn.__name__, level)
    x1 = A.quantize_activation(x[:1].contiguous(), refine=True, exclude_mask=wp.mask)
    assert torch.equal(A.gemv(wp, x1, bits=6), A.gemv(got["w"], x1, bits=6))


@pytest.mark.parametrize("name,b", [("wgate", 1), ("wgate", 8), ("wdown", 8), ("wqkv", 1), ("wqkv", 8), ("wqkv", 16),
                                    ("wdown", 64), ("wqkv", 64), ("wgate", 64)])
def test_full_size_decode_sampled(name, b):
    """Llama-3-8B-shaped layer at full size: every output of sampled weight
    rows checked against the oracle at levels 2 and 4 (and 6 on Wqkv)."""
    n, k = S.LLAMA8B[name]
    say(f"case: full-size {name} {n}x{k} batch {b}")
    w = S.weights(n, k, seed=1, tensor_id=list(S.LLAMA8B).index(name), device=DEV)
    x = S.activations(b, k, seed=1, tensor_id=99, device=DEV)
    levels = (2, 4, 6) if name == "wqkv" else (2, 4)
    wp = A.quantize_weight(w, refine=(6 in levels))
    xp4 = A.quantize_activation(x)
    xn = x.float().cpu().numpy()
    rows = np.random.default_rng(2).choice(n, 64, replace=False)
    wn = w.cpu().numpy()
    amax = np.abs(wn).max()
    if 6 in levels:
        bits, _ = O.select_weight_mask(wn, 0.2)
        wq = O.quantize_weight(wn[rows], O.pack_nibbles(bits), tensor_amax=amax)
        xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
        xq6 = O.quantize_activation(xn, refine=True, exclude_mask=wq["mask"])
    else:
        wq = O.quantize_weight(wn[rows], tensor_amax=amax)
        xp6 = xq6 = None
    xq4 = O.quantize_activation(xn)
    for level in levels:
        y = A.gemv(wp, xp6 if level == 6 else xp4, bits=level).cpu().numpy()
        ref = O.linear(wq, xq6 if level == 6 else xq4, level)
        check_close(y[:, rows], ref)


@pytest.mark.parametrize("name,n,k", [("wo", 4096, 4096), ("wdown", 4096, 14336), ("wgateup", 28672, 4096)])
def test_full_size_one_token_all_levels(name, n, k):
    """The one-token launches the decode benchmark times, at full size and at
    all three levels (the fused Wgate|Wup is one 28672 x 4096 weight): every
    output of 64 sampled weight rows, the first and last among them, against
    the oracle. The oracle selects M_W over the whole weight."""
    say(f"case: full-size one token {name} {n}x{k}")
    w = S.weights(n, k, seed=3, tensor_id=7, device=DEV)
    x = S.activations(1, k, seed=3, tensor_id=98, device=DEV)
    wp = A.quantize_weight(w, refine=True)
    xp4 = A.quantize_activation(x)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
    wn = w.cpu().numpy()
    xn = x.float().cpu().numpy()
    rows = np.concatenate([[0, n - 1], np.random.default_rng(4).choice(np.arange(1, n - 1), 62, replace=False)])
    bits, _ = O.select_weight_mask(wn, 0.2)
    wq = O.quantize_weight(wn[rows], O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    xq4 = O.quantize_activation(xn)
    xq6 = O.quantize_activation(xn, refine=True, exclude_mask=wq["mask"])
    for level in (2, 4, 6):
        y = A.gemv(wp, xp6 if level == 6 else xp4, bits=level).cpu().numpy()
        check_close(y[:, rows], O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("b", [16, 64])
def test_full_size_70b_gemv_sampled(b):
    """The 70B-shaped projection (28672 x 8192) at 16 and 64 tokens, levels 2
    and 4: every output of 64 sampled weight rows against the oracle."""
    n, k = 28672, 8192
    say(f"case: full-size 70B GEMV {n}x{k} batch {b}")
    w = S.weights(n, k, seed=3, tensor_id=70, device=DEV)
    x = S.activations(b, k, seed=3, tensor_id=71, device=DEV)
    wp = A.quantize_weight(w)
    xp4 = A.quantize_activation(x)
    rows = np.random.default_rng(5).choice(n, 64, replace=False)
    wn = w.cpu().numpy()
    wq = O.quantize_weight(wn[rows], tensor_amax=np.abs(wn).max())
    xq4 = O.quantize_activation(x.float().cpu().numpy())
    del w, wn
    for level in (2, 4):
        y = A.gemv(wp, xp4, bits=level).cpu().numpy()
        check_close(y[:, rows], O.linear(wq, xq4, level))


@pytest.mark.parametrize("name", ["wup", "wdown"])
def test_prefill_sampled_full_size(name):
    """The prefill GEMMs the benchmark times, at full size, levels 4 and 6:
    2048 x 4096 activations times Wup (14336 x 4096), and the FFN output
    X' (2048 x 14336) times Wdown (4096 x 14336, 224 K steps of the 256 x 128
    tile). Sampled tokens and weight rows (the first and last of each among
    them) against the oracle."""
    n, k = S.LLAMA8B[name]
    m = 2048
    say(f"case: full-size prefill GEMM {name} {m}x{k}x{n}")
    w = S.weights(n, k, seed=2, tensor_id=5 if name == "wup" else 8, device=DEV)
    x = S.activations(m, k, seed=2, tensor_id=6 if name == "wup" else 9, outlier_frac=0.005,
                      outlier_scale=30.0, device=DEV)
    wp = A.quantize_weight(w, refine=True)
    xp4 = A.quantize_activation(x)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
    rng = np.random.default_rng(3)
    rows = np.concatenate([[0, n - 1], rng.choice(np.arange(1, n - 1), 30, replace=False)])
    toks = np.concatenate([[0, m - 1], rng.choice(np.arange(1, m - 1), 30, replace=False)])
    wn = w.cpu().numpy()
    xn = x.float().cpu().numpy()
    bits, _ = O.select_weight_mask(wn, 0.2)
    wq = O.quantize_weight(wn[rows], O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    xa = np.abs(xn).max()
    for level, xp in ((4, xp4), (6, xp6)):
        xq = O.quantize_activation(xn[toks], refine=(level == 6), exclude_mask=wq["mask"], tensor_amax=xa)
        y = A.gemm(wp, xp, bits=level).cpu().numpy()
        e = check_close(y[np.ix_(toks, rows)], O.linear(wq, xq, level))
        say(f"level {level}: max rel err {e:.2e}")


def test_prefill_activation_panel_beyond_2gib():
    """75000 prefill tokens at K = 14336: the fp16 activation panel in the
    workspace holds 75000 x 14336 x 2 = 2.15e9 bytes, past 2^31, so tokens
    74899 .. 74999 lie beyond the reach of one 32-bit buffer offset from the
    panel's start. Sampled tokens on both sides of that point (the first and
    the last token among them) at levels 4 and 6 against the oracle; the
    oracle takes the tensor scale of the whole activation (its absolute
    maximum, found on the host)."""
    n, k, m = 256, 14336, 75000
    say(f"case: prefill GEMM {m}x{k}x{n}, activation panel past 2^31 bytes")
    assert m * k * 2 > 2 ** 31
    w = S.weights(n, k, seed=4, tensor_id=11, device=DEV)
    x = S.activations(m, k, seed=4, tensor_id=12, outlier_frac=0.005, outlier_scale=30.0, device=DEV)
    wp = A.quantize_weight(w, refine=True)
    xp4 = A.quantize_activation(x)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=wp.mask)
    first_far = -(-2 ** 31 // (k * 2))                # first token whose panel row starts past 2^31
    rng = np.random.default_rng(13)
    toks = np.unique(np.concatenate([[0, 1, first_far - 1, first_far, m - 1],
                                     rng.choice(m, 20, replace=False),
                                     rng.choice(np.arange(first_far, m), 10, replace=False)]))
    x_host = x.cpu()
    xa = np.float32(x_host.abs().max().float().item())
    xn = x_host[torch.from_numpy(toks)].float().numpy()
    del x_host, x
    wn = w.cpu().numpy()
    bits, _ = O.select_weight_mask(wn, 0.2)
    wq = O.quantize_weight(wn, O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    for level, xp in ((4, xp4), (6, xp6)):
        say(f"level {level}")
        y = A.gemm(wp, xp, bits=level)
        ys = y[torch.from_numpy(toks).to(DEV)].cpu().numpy()
        del y
        xq = O.quantize_activation(xn, refine=(level == 6), exclude_mask=wq["mask"], tensor_amax=xa)
        e = check_close(ys, O.linear(wq, xq, level))
        say(f"level {level}: max rel err {e:.2e}")
    del xp4, xp6
    torch.cuda.empty_cache()


def _budget_mask(k, R, seed):
    """A valid weight mask chosen by the test: R refined subgroups spread at
    random over the 16-element groups, at most two per group (returned as one
    4-bit value per group). GEMV parity does not depend on how M_W was
    selected; the selection has tests of its own."""
    rng = np.random.default_rng(seed)
    G = k // 16
    nib = np.zeros(G, np.uint8)
    for slot in rng.permutation(2 * G)[:R]:
        g = slot // 2
        free = [b for b in range(4) if not (int(nib[g]) >> b) & 1]
        nib[g] |= np.uint8(1 << int(rng.choice(free)))
    return nib


@pytest.mark.parametrize("b", [16, 64])
def test_full_size_70b_gemv_level6(b):
    """The 70B-shaped projection (28672 x 8192) at 16 and 64 tokens, level 6
    (the 64-token tile refines both operands): every output of 64 sampled
    weight rows, the first and last among them, against the oracle."""
    n, k = 28672, 8192
    say(f"case: full-size 70B GEMV {n}x{k} batch {b}, level 6")
    w = S.weights(n, k, seed=3, tensor_id=70, device=DEV)
    x = S.activations(b, k, seed=3, tensor_id=71, device=DEV)
    R = A.weight_refined_count(k)
    nib = _budget_mask(k, R, seed=6)
    assert sum(bin(int(v)).count("1") for v in nib) == R
    mask_np = O.pack_nibbles(nib)
    mask = torch.from_numpy(mask_np).to(DEV)
    wp = A.quantize(w, N.WEIGHT, weight_mask=mask, n_refined=R)
    xp6 = A.quantize_activation(x, refine=True, exclude_mask=mask)
    rows = np.concatenate([[0, n - 1], np.random.default_rng(5).choice(np.arange(1, n - 1), 62, replace=False)])
    wn = w.cpu().numpy()
    wq = O.quantize_weight(wn[rows], mask_np, tensor_amax=np.abs(wn).max())
    xq6 = O.quantize_activation(x.float().cpu().numpy(), refine=True, exclude_mask=mask_np)
    del w, wn
    y = A.gemv(wp, xp6, bits=6).cpu().numpy()
    e = check_close(y[:, rows], O.linear(wq, xq6, 6))
    say(f"max rel err {e:.2e}")


def _all_scale_codes_weight(n, k, seed):
    """Weights whose 16-element groups span the whole E4M3 scale range: each
    group's absolute maximum is 2^u with u uniform in [-17, 0] (one element set
    to +-that value, one row holding 1.0), so B = E4M3(448 * amax_j / amax)
    takes codes from the subnormal range up to 448."""
    rng = np.random.default_rng(seed)
    g = k // 16
    amax_g = np.exp2(rng.uniform(-17.0, 0.0, (n, g)))
    amax_g[0, 0] = 1.0
    w = rng.uniform(-1.0, 1.0, (n, g, 16)) * amax_g[:, :, None]
    w[:, :, 0] = np.where(rng.random((n, g)) < 0.5, -1.0, 1.0) * amax_g
    return w.reshape(n, k).astype(np.float32)


@pytest.mark.parametrize("level", [2, 4, 6])
@pytest.mark.parametrize("b", [1, 5])
def test_gemv_all_scale_codes(level, b):
    """Every E4M3 group-scale code range (subnormal to 448) through the GEMV's
    scale conversion."""
    say(f"case: gemv all scale codes level {level} B={b}")
    n, k = 48, 19 * 16 * 8
    wn = _all_scale_codes_weight(n, k, seed=11)
    w = torch.from_numpy(wn).to(DEV)
    x = S.activations(b, k, seed=12, tensor_id=0, device=DEV)
    wp, xp4, xp6 = gpu_pack(w, x)
    codes = set(np.unique(wp.scales.cpu().numpy()).tolist())
    assert len(codes) >= 100, len(codes)
    wq, xq4, xq6 = oracle_pack(w, x)
    y = run(A.gemv, wp, xp4, xp6, level)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("n,b,k,waves", [(33024, 1, 512, 0), (33024, 3, 768, 1), (8192, 2, 1024, 4)])
def test_gemv_many_tiles(n, b, k, waves):
    """Enough row tiles that the kernel keeps 4 rather than 8 chunks in flight
    per wavefront (more than 2048 wavefronts), against the oracle."""
    say(f"case: gemv many tiles N={n} B={b} K={k} waves={waves}")
    w, x = operands(n, b, k, seed=n + k)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    p = A.default_params(gemv_waves=waves)
    for level in (2, 4, 6):
        y = run(A.gemv, wp, xp4, xp6, level, params=p)
        check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("n,b,k", [(8200, 64, 448), (8256, 17, 64 * 9), (12300, 40, 64 * 5), (8192, 33, 64),
                                   (16448, 20, 64 * 3)])
def test_gemv_batched_k_groups(n, b, k):
    """17-64 tokens on weights of 8192+ rows: the 64-token tile whose wavefront
    groups each take a share of the K steps (four groups below 256 row tiles,
    two from 256: 16448 rows), with step counts that do not divide evenly, a
    single step and ragged row tiles, against the oracle at every level."""
    say(f"case: batched gemv K groups N={n} B={b} K={k}")
    w, x = operands(n, b, k, seed=n + b + k)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    for level in (2, 4, 6):
        y = run(A.gemv, wp, xp4, xp6, level)
        check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("waves", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n,b,k", [(40, 1, 4096 + 256), (33, 3, 2304 + 64), (16, 16, 1040)])
def test_gemv_forced_waves(waves, n, b, k):
    """The GEMV at every wavefront count; with one wavefront per tile and
    K = 4352 a wavefront walks 17 chunks (two rounds of its offset plan)."""
    say(f"case: gemv waves={waves} N={n} B={b} K={k}")
    w, x = operands(n, b, k, seed=waves * 31 + n)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    p = A.default_params(gemv_waves=waves)
    for level in (2, 4, 6):
        y = run(A.gemv, wp, xp4, xp6, level, params=p)
        check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("n,k,waves", [(200, 256, 0), (1000, 4096, 0), (17, 2560, 1), (33, 768, 2),
                                       (300, 14336, 0), (40, 4096 + 256, 16), (16400, 256, 0)])
@pytest.mark.parametrize("level", [2, 4, 6])
def test_gemv_one_token_matrix_core_path(n, k, waves, level):
    """One token with K % 256 == 0 (the fp4 matrix-core GEMV): ragged row
    tiles, uneven and forced K splits, host- and device-side level; 16400
    rows (1025 row tiles) takes the whole-row loads at levels 2 and 4."""
    say(f"case: one-token gemv N={n} K={k} waves={waves} level {level}")
    w, x = operands(n, 1, k, seed=n + k + waves)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    p = A.default_params(gemv_waves=waves)
    y = run(A.gemv, wp, xp4, xp6, level, params=p)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))
    yb = run(A.gemv, wp, xp4, xp6, level, params=p, out_dtype=torch.bfloat16)
    assert torch.equal(yb, y.to(torch.bfloat16)), "bf16 output is not the RNE of the fp32 result"
    dev_bits = torch.tensor([level], dtype=torch.int32, device=DEV)
    yd = A.gemv(wp, xp6, bits=0, bits_dev=dev_bits, params=p)   # refinement unused below level 6
    assert torch.equal(yd, y), "device-side level differs from the host-given level"


@pytest.mark.parametrize("n,b,k,waves", [(200, 2, 256, 0), (1000, 3, 4096, 0), (64, 4, 2560, 1),
                                         (300, 5, 14336, 0), (40, 8, 4352, 0), (33, 7, 768, 2),
                                         (16400, 8, 256, 0), (9000, 2, 1024, 0)])
@pytest.mark.parametrize("level", [2, 4, 6])
def test_gemv_few_tokens_matrix_core_path(n, b, k, waves, level):
    """2-8 tokens with K % 256 == 0: two tokens per MFMA (one token's codes
    and offsets at level 6, which takes up to 4 tokens); odd token counts
    leave A rows empty; host- and device-side level; bf16 output."""
    say(f"case: few-token gemv N={n} B={b} K={k} waves={waves} level {level}")
    w, x = operands(n, b, k, seed=n + 7 * b + k + waves)
    wp, xp4, xp6 = gpu_pack(w, x)
    wq, xq4, xq6 = oracle_pack(w, x)
    p = A.default_params(gemv_waves=waves)
    y = run(A.gemv, wp, xp4, xp6, level, params=p)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))
    yb = run(A.gemv, wp, xp4, xp6, level, params=p, out_dtype=torch.bfloat16)
    assert torch.equal(yb, y.to(torch.bfloat16)), "bf16 output is not the RNE of the fp32 result"
    dev_bits = torch.tensor([level], dtype=torch.int32, device=DEV)
    yd = A.gemv(wp, xp6, bits=0, bits_dev=dev_bits, params=p)
    check_close(yd.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))


@pytest.mark.parametrize("n,k", [(64, 4096), (48, 1024)])
def test_gemv_one_token_overlapping_refinement(n, k):
    """Activation refined in subgroups the weight also refines (no exclusion
    mask): the product needs the d_W * d_A / 64 term too."""
    say(f"case: one-token gemv overlapping refinement N={n} K={k}")
    w, x = operands(n, 1, k, seed=n * 3 + k)
    wp = A.quantize_weight(w, refine=True)
    xp = A.quantize_activation(x, refine=True)
    wq, _, _ = oracle_pack(w, x)
    xq = O.quantize_activation(x.float().cpu().numpy(), refine=True)
    both = (wq["mask"][None, :] & xq["mask"]).any()
    assert both, "the case needs subgroups refined on both sides"
    y = A.gemv(wp, xp, bits=6)
    check_close(y.cpu().numpy(), O.linear(wq, xq, 6))


@pytest.mark.parametrize("level", [2, 4, 6])
def test_gemv_one_token_all_scale_codes(level):
    """Every E4M3 scale range through the one-token matrix-core GEMV (scales
    applied in fp32 to exact per-group dot products)."""
    say(f"case: one-token gemv all scale codes level {level}")
    n, k = 48, 2560
    wn = _all_scale_codes_weight(n, k, seed=13)
    w = torch.from_numpy(wn).to(DEV)
    x = S.activations(1, k, seed=14, tensor_id=0, device=DEV)
    wp, xp4, xp6 = gpu_pack(w, x)
    assert len(set(np.unique(wp.scales.cpu().numpy()).tolist())) >= 100
    wq, xq4, xq6 = oracle_pack(w, x)
    y = run(A.gemv, wp, xp4, xp6, level)
    check_close(y.cpu().numpy(), O.linear(wq, xq6 if level == 6 else xq4, level))
