"""GPU parity of the producer epilogue (autofp_epilogue_quantize): the layer's
elementwise step on a completed linear output (copy of the first k columns,
residual add, SwiGLU) fused with the AutoFP encode of the result into the
next layer's activation ([AE] §6.4).

  - v (written to v_out) against the oracle's fp64 epilogue: bit for bit for
    copy and residual (one fp32 rounding of an exact sum), within 2e-6
    relative for SwiGLU (fp32 exp and division);
  - the packed output bit for bit against the oracle's encode of that same v
    (the encode of a given fp32 tensor is exact), at 1 token (one launch), 4
    and 64 tokens, with and without refinement and an exclusion mask;
  - and against autofp_quantize of v, byte for byte;
  - autofp_layer_epilogue (the residual RMSNorm epilogue with the layer's L_A
    and policy step in the same launch) against the epilogue followed by
    autofp_policy_layer: hidden state, bytes, L_A, levels and state equal
    over a sequence of layers and steps.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same_packed(gpu, ref, refine):
    h = gpu.to_host()
    keys = ("codes", "scales", "mask", "offsets") if refine else ("codes", "scales")
    for key in keys:
        assert np.array_equal(h[key], ref[key]), key
    assert np.float32(h["T"]) == np.float32(ref["T"])


@pytest.mark.parametrize("op", ["copy", "residual", "swiglu"])
@pytest.mark.parametrize("rows,k", [(1, 4096), (4, 4096), (8, 4096), (1, 14336), (2, 14336), (64, 1024), (3, 272)])
@pytest.mark.parametrize("refine", [False, True])
def test_epilogue_quantize(op, rows, k, refine):
    say(f"case: epilogue {op} rows={rows} k={k} refine={refine}")
    ldz = (2 * k if op == "swiglu" else k + 256)
    z = S.hidden(rows, ldz, seed=rows + k, tensor_id=1, device=DEV) * 3.0
    resid = S.hidden(rows, k, seed=rows + k, tensor_id=2, device=DEV)
    wm, _ = A.select_weight_mask(S.weights(64, k, seed=3, tensor_id=3, device=DEV))
    ex = wm if refine else None
    out = A.alloc_activation(rows, k, refine=refine, device=DEV)
    v = torch.empty(rows, k, dtype=torch.float32, device=DEV)
    A.epilogue_quantize(op, z, out, residual=resid if op == "residual" else None, v_out=v,
                        refine=refine, exclude_mask=ex)
    torch.cuda.synchronize()
    vg = v.cpu().numpy()
    vr = O.epilogue(op, z.cpu().numpy(), k, resid.cpu().numpy())
    if op == "swiglu":
        rel = np.abs(vg - vr) / np.maximum(np.abs(vr), 1e-30)
        assert rel.max() <= 2e-6, rel.max()
    else:
        assert np.array_equal(vg, vr.astype(np.float32))
    exn = None if ex is None else ex.cpu().numpy()
    ref = O.quantize_activation(vg, refine=refine, exclude_mask=exn)
    same_packed(out, ref, refine)
    # the separate encode of the same v gives the same bytes
    q = A.quantize_activation(v, refine=refine, exclude_mask=ex)
    torch.cuda.synchronize()
    for key in ("codes", "scales", "tensor_scale") + (("mask", "offsets") if refine else ()):
        assert torch.equal(getattr(q, key), getattr(out, key)), key


def test_epilogue_without_v_out_and_arguments():
    rows, k = 2, 512
    z = S.hidden(rows, 2 * k, seed=9, tensor_id=1, device=DEV)
    out = A.alloc_activation(rows, k, refine=False, device=DEV)
    A.epilogue_quantize("swiglu", z, out)
    ref = O.quantize_activation(np.asarray(O.epilogue("swiglu", z.cpu().numpy(), k), np.float32))
    # v is recomputed in fp32 on the device: compare through the device's own v
    v = torch.empty(rows, k, dtype=torch.float32, device=DEV)
    out2 = A.alloc_activation(rows, k, refine=False, device=DEV)
    A.epilogue_quantize("swiglu", z, out2, v_out=v)
    torch.cuda.synchronize()
    assert torch.equal(out.codes, out2.codes) and torch.equal(out.scales, out2.scales)
    assert ref["codes"].shape == out.to_host()["codes"].shape
    with pytest.raises(A.AutofpError):
        A.epilogue_quantize("swiglu", z[:, :k + 16].contiguous(), out)      # ldz < 2k
    with pytest.raises(A.AutofpError):
        A.epilogue_quantize("residual", z, out)                             # residual missing


@pytest.mark.parametrize("rows,k", [(1, 4096), (4, 4096), (8, 4096), (1, 14336), (2, 14336), (3, 272), (64, 1024), (64, 4096), (16, 14336)])
@pytest.mark.parametrize("refine", [False, True])
def test_epilogue_residual_rmsnorm(rows, k, refine):
    """Residual add + RMSNorm (one launch up to 4096 subgroup slots: 1 x 4096,
    4 x 4096, 1 x 14336, 3 x 272; the row-scale pass above: 64 x 1024,
    64 x 4096, 16 x 14336): v_out holds u = residual + z bit for bit; the
    packed output equals the oracle's encode of the oracle's normalized v
    (whose row scales are fp32 roundings of fp64 sums) bit for bit, and the
    device encode of that same v byte for byte. The rows carry different
    scales (one of them 1e3 larger, one small enough for eps to matter)."""
    say(f"case: epilogue residual_rmsnorm rows={rows} k={k} refine={refine}")
    ldz = k + 256
    z = S.hidden(rows, ldz, seed=rows + k, tensor_id=5, device=DEV) * 3.0
    resid = S.hidden(rows, k, seed=rows + k, tensor_id=6, device=DEV)
    if rows > 1:
        resid[0] *= 1e3
        z[0] *= 1e3
        resid[-1] *= 1e-3
        z[-1] *= 1e-3
    wm, _ = A.select_weight_mask(S.weights(64, k, seed=3, tensor_id=3, device=DEV))
    ex = wm if refine else None
    out = A.alloc_activation(rows, k, refine=refine, device=DEV)
    u = torch.empty(rows, k, dtype=torch.float32, device=DEV)
    A.epilogue_quantize("residual_rmsnorm", z, out, residual=resid, v_out=u, refine=refine, exclude_mask=ex)
    torch.cuda.synchronize()
    v_ref, u_ref = O.rmsnorm_residual(z.cpu().numpy(), k, resid.cpu().numpy())
    assert np.array_equal(u.cpu().numpy(), u_ref)
    exn = None if ex is None else ex.cpu().numpy()
    ref = O.quantize_activation(v_ref, refine=refine, exclude_mask=exn)
    same_packed(out, ref, refine)
    q = A.quantize_activation(torch.from_numpy(v_ref).to(DEV), refine=refine, exclude_mask=ex)
    torch.cuda.synchronize()
    for key in ("codes", "scales", "tensor_scale") + (("mask", "offsets") if refine else ()):
        assert torch.equal(getattr(q, key), getattr(out, key)), key
    # deterministic: a second call gives the same bytes
    out2 = A.alloc_activation(rows, k, refine=refine, device=DEV)
    A.epilogue_quantize("residual_rmsnorm", z, out2, residual=resid, refine=refine, exclude_mask=ex)
    torch.cuda.synchronize()
    assert torch.equal(out2.codes, out.codes) and torch.equal(out2.tensor_scale, out.tensor_scale)


@pytest.mark.parametrize("rows,k", [(1, 4096), (4, 4096), (8, 4096), (3, 1024), (16, 4096)])
@pytest.mark.parametrize("phase", [1, 0])
def test_layer_epilogue_equals_epilogue_then_policy_layer(rows, k, phase):
    """autofp_layer_epilogue (the residual RMSNorm epilogue with the layer's
    L_A and Table 1 step fused: one launch up to 16384 elements, the two
    calls above) against autofp_epilogue_quantize("residual_rmsnorm")
    followed by autofp_policy_layer, over 3 steps x 6 layers of a sequence
    with two policy states evolving side by side: v_out and the encoded bytes
    bit for bit, L_A, the levels, the layer maximum and the whole state equal
    after every layer. The update sizes vary by layer and step so the trend
    counters move both ways; G_E straddles tau = 0.1 in decode."""
    say(f"case: layer epilogue rows={rows} k={k} phase={phase}")
    wm, _ = A.select_weight_mask(S.weights(64, k, seed=5, tensor_id=3, device=DEV))
    st_a, st_b = A.policy_state(rows, DEV), A.policy_state(rows, DEV)
    ws_a = torch.empty(A.workspace_bytes(A.N.OP_EPILOGUE, rows, k), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty_like(ws_a)
    h_prev = S.hidden(rows, k, seed=11, tensor_id=0, device=DEV)
    for step in range(3):
        g_e = torch.tensor([0.05 + 0.1 * ((r + step) % 3) for r in range(rows)], dtype=torch.float32, device=DEV)
        for layer in range(6):
            scale = 0.02 * (1 + ((layer * 7 + step * 3) % 5))
            z = S.hidden(rows, k + 64, seed=100 * step + layer, tensor_id=1, device=DEV) * scale
            resid = (h_prev + S.hidden(rows, k, seed=100 * step + layer, tensor_id=2, device=DEV) * scale).contiguous()
            out_a = A.alloc_activation(rows, k, refine=True, device=DEV)
            out_b = A.alloc_activation(rows, k, refine=True, device=DEV)
            v_a = torch.empty(rows, k, dtype=torch.float32, device=DEV)
            v_b = torch.empty_like(v_a)
            new_seq = step == 0 and layer == 0
            ge = g_e if phase == 1 else None
            A.epilogue_quantize("residual_rmsnorm", z, out_a, residual=resid, v_out=v_a, refine=True,
                                exclude_mask=wm, workspace=ws_a)
            la_a, br_a, bl_a = A.policy_layer(phase, layer, h_prev, v_a, st_a, g_e=ge, new_sequence=new_seq)
            la_b, br_b, bl_b = A.layer_epilogue(z, out_b, resid, v_b, h_prev, phase, layer, st_b, g_e=ge,
                                                new_sequence=new_seq, refine=True, exclude_mask=wm, workspace=ws_b)
            torch.cuda.synchronize()
            assert torch.equal(v_a, v_b)
            for key in ("codes", "scales", "tensor_scale", "mask", "offsets"):
                assert torch.equal(getattr(out_a, key), getattr(out_b, key)), key
            assert torch.equal(la_a, la_b), (step, layer, la_a, la_b)
            assert torch.equal(br_a, br_b) and torch.equal(bl_a, bl_b), (step, layer)
            assert torch.equal(st_a, st_b), (step, layer)
            h_prev = v_a.clone()
