"""GPU parity of the AutoFP encoder and weight-mask selection (bit-exact)."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import synthetic as S
from conftest import read_golden

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_same_packed(gpu: A.AutoFPTensor, ref: dict, fields=("codes", "scales", "T", "mask", "offsets")):
    h = gpu.to_host()
    for f in fields:
        if f not in ref:
            continue
        a, b = np.asarray(h[f]), np.asarray(ref[f])
        if f == "T":
            assert np.float32(a) == np.float32(b), (f, a, b)
        else:
            assert a.shape == b.shape, (f, a.shape, b.shape)
            diff = np.argwhere(a != b)
            assert diff.size == 0, (f, diff[:5].tolist(), a[tuple(diff[0])], b[tuple(diff[0])])


def test_table7_group_on_gpu():
    rows = read_golden("table7_group.txt")
    xs = np.array([float(r[0]) for r in rows], np.float32) * np.float32(0.25)
    x = torch.from_numpy(xs.reshape(1, 16)).to(DEV)
    say("case: Table 7 group, activation refine")
    pk = A.quantize_activation(x, refine=True)
    h = pk.to_host()
    codes = O.unpack_nibbles(h["codes"], 16)[0]
    assert [int(c) for c in codes] == [int(r[2], 2) for r in rows]
    assert int(h["scales"][0, 0]) == 0x7E
    assert int(h["mask"][0, 0]) == 0b0110
    for i, r in enumerate(rows):
        byte = int(h["offsets"][0, i // 4])
        d = (byte >> (2 * (i % 4))) & 3
        assert d == (int(r[4], 2) if r[3] == "1" else 0), i


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("refine", [False, True])
def test_activation_encode_config1(dtype, refine):
    say(f"case: C1 activations 16x256 {dtype} refine={refine}")
    x = S.activations(16, 256, seed=0, tensor_id=1, outlier_frac=0.01, outlier_scale=20.0,
                      dtype=dtype, device=DEV)
    w = S.weights(256, 256, seed=0, tensor_id=2, heavy_frac=0.0, device=DEV)
    wmask, _ = A.select_weight_mask(w)
    pk = A.quantize_activation(x, refine=refine, exclude_mask=wmask if refine else None)
    ref = O.quantize_activation(x.float().cpu().numpy(), refine=refine,
                                exclude_mask=wmask.cpu().numpy() if refine else None)
    assert_same_packed(pk, ref)


@pytest.mark.parametrize("shape", [(1, 4096), (4, 4096), (5, 4096), (8, 4096), (9, 4096), (1, 14336), (2, 14336),
                                   (3, 14336), (64, 16), (65, 16), (128, 16), (129, 16), (32, 272), (33, 272),
                                   (64, 272), (65, 272), (8, 14336), (8192, 16), (8193, 16), (16, 14336), (3, 65536)])
def test_activation_encode_one_and_two_launch_paths(shape):
    """Decode-step activation shapes on both sides of the single-launch limits
    (rows * roundup(k/4, 64) subgroup slots: 256-thread blocks up to 4096 —
    4 x 4096, 64 x 16, 32 x 272 —, 512-thread blocks up to 8192 — 8 x 4096,
    2 x 14336, 128 x 16, 64 x 272 —, one row more takes the next form):
    bit-exact codes, scales, T, mask and offsets."""
    rows, k = shape
    say(f"case: activation encode {rows}x{k} (bf16, refine, exclusion mask)")
    x = S.activations(rows, k, seed=rows + k, tensor_id=3, dtype=torch.bfloat16, device=DEV)
    g = torch.Generator().manual_seed(k)
    excl = torch.randint(0, 256, ((k + 31) // 32,), generator=g, dtype=torch.uint8).to(DEV)
    pk = A.quantize_activation(x, refine=True, exclude_mask=excl)
    ref = O.quantize_activation(x.float().cpu().numpy(), refine=True, exclude_mask=excl.cpu().numpy())
    assert_same_packed(pk, ref)
    pk4 = A.quantize_activation(x, refine=False)
    assert_same_packed(pk4, O.quantize_activation(x.float().cpu().numpy(), refine=False))


@pytest.mark.parametrize("shape,rho", [((256, 256), 0.2), ((48, 272), 0.2), ((300, 512), 0.35),
                                       ((7, 32), 0.5)])
def test_weight_mask_and_encode(shape, rho):
    say(f"case: weight mask+encode {shape} rho={rho}")
    n, k = shape
    w = S.weights(n, k, seed=3, tensor_id=n + k, device=DEV)
    p = A.default_params(rho=rho)
    pk = A.quantize_weight(w, refine=True, params=p)
    wn = w.cpu().numpy()
    bits, R = O.select_weight_mask(wn, rho)
    assert pk.n_refined == R
    ref = O.quantize_weight(wn, O.pack_nibbles(bits))
    assert_same_packed(pk, ref)


def _edge_inputs():
    rng = np.random.default_rng(7)
    cases = {}
    cases["zeros"] = np.zeros((3, 64), np.float32)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    x[0, 16:32] *= 1e-6                       # group scale underflows
    x[1, 32:48] = 0.0                         # zero group
    x[2, :16] = 0.96 * np.abs(x).max()        # scale rounds down, values saturate
    cases["tiny_zero_saturate"] = x
    mid = 0.25 * (rng.integers(-24, 25, (5, 64)) / 4.0)
    mid[:, 0] = 1.5
    cases["midpoint_ties"] = mid.astype(np.float32)
    cases["k_mod_32_is_16"] = rng.standard_normal((9, 272)).astype(np.float32)
    cases["single_row"] = rng.standard_normal((1, 16)).astype(np.float32) * 1e3
    cases["many_rows"] = (rng.standard_normal((1000, 96)) * np.exp2(rng.integers(-8, 8, (1000, 96)))).astype(np.float32)
    return cases


@pytest.mark.parametrize("name", list(_edge_inputs().keys()))
def test_encode_edge_cases(name):
    say(f"case: encode edge {name}")
    xn = _edge_inputs()[name]
    x = torch.from_numpy(xn).to(DEV)
    pk = A.quantize_activation(x, refine=True)
    assert_same_packed(pk, O.quantize_activation(xn, refine=True))
    pkw = A.quantize_weight(x, refine=xn.shape[1] >= 32)
    if xn.shape[1] >= 32:
        bits, _ = O.select_weight_mask(xn, 0.2)
        assert_same_packed(pkw, O.quantize_weight(xn, O.pack_nibbles(bits)))
    else:
        assert_same_packed(pkw, O.quantize_weight(xn))


def test_encode_is_deterministic():
    say("case: encode determinism")
    x = S.activations(64, 4096, seed=5, tensor_id=0, device=DEV)
    a = A.quantize_activation(x, refine=True).to_host()
    b = A.quantize_activation(x, refine=True).to_host()
    for f in ("codes", "scales", "mask", "offsets"):
        assert (a[f] == b[f]).all()
    assert a["T"] == b["T"]


def test_full_size_weight_sampled_rows():
    """Wo 4096x4096 (Llama-3-8B shape): mask over the whole tensor, codes and
    offsets of sampled rows, all bit-exact."""
    say("case: full-size Wo 4096x4096 mask + sampled rows")
    w = S.weights(4096, 4096, seed=0, tensor_id=11, device=DEV)
    pk = A.quantize_weight(w, refine=True)
    wn = w.cpu().numpy()
    bits, R = O.select_weight_mask(wn, 0.2)
    assert pk.mask.cpu().numpy().tolist() == O.pack_nibbles(bits).tolist()
    rows = np.random.default_rng(1).choice(4096, 48, replace=False)
    ref = O.quantize_weight(wn[rows], O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    h = pk.to_host()
    assert np.float32(h["T"]) == np.float32(ref["T"])
    assert (h["codes"][rows] == ref["codes"]).all()
    assert (h["scales"][rows] == ref["scales"]).all()
    assert (h["offsets"][rows] == ref["offsets"]).all()


def test_many_rows_weight_encode_row_loop():
    """More rows than encoder blocks along the row axis (each block encodes
    several rows): codes, scales and compacted offsets of sampled rows."""
    say("case: weight encode 20000x256, rows looped per block")
    w = S.weights(20000, 256, seed=4, tensor_id=5, device=DEV)
    pk = A.quantize_weight(w, refine=True)
    wn = w.cpu().numpy()
    bits, _ = O.select_weight_mask(wn, 0.2)
    rows = np.sort(np.random.default_rng(2).choice(20000, 64, replace=False))
    rows[-1] = 19999
    ref = O.quantize_weight(wn[rows], O.pack_nibbles(bits), tensor_amax=np.abs(wn).max())
    h = pk.to_host()
    assert np.float32(h["T"]) == np.float32(ref["T"])
    for f in ("codes", "scales", "offsets"):
        assert (h[f][rows] == ref[f]).all(), f
