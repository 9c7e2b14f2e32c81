"""autofp_quantize_noalloc (static per-GPU scratch, no workspace argument)
against autofp_quantize (caller workspace) on the same inputs, byte for byte,
on calls in a row whose sizes shrink, so every call after the first finds the
previous call's contents in the scratch array."""

import sys

import pytest
import torch

import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import _native as N
from runtime_mixed_precision_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same(a, b, what):
    for name in ("codes", "scales", "tensor_scale", "mask", "offsets"):
        fa, fb = getattr(a, name), getattr(b, name)
        assert (fa is None) == (fb is None), (what, name)
        if fa is not None:
            assert torch.equal(fa, fb), (what, name)


def test_noalloc_quantize_equals_workspace_quantize():
    # 1: a weight with its mask (amax partials of 58.7M elements, mask prefix table)
    say("case: noalloc weight 4096x14336 fp32 with mask")
    w = S.weights(4096, 14336, seed=7, tensor_id=1, device=DEV)
    mask, nref = A.select_weight_mask(w)
    ref = A.quantize(w, N.WEIGHT, weight_mask=mask, n_refined=nref)
    out = A._alloc_packed(4096, 14336, N.WEIGHT, True, nref, DEV)
    out.mask = mask
    A.quantize_noalloc(w, out)
    torch.cuda.synchronize()
    same(out, ref, "weight 4096x14336")
    del w

    # 2: smaller - a refined activation of 300 tokens (fewer partials, stale ones after them)
    say("case: noalloc activation 300x4096 bf16, refined")
    wm, _ = A.select_weight_mask(S.weights(64, 4096, seed=7, tensor_id=3, device=DEV))
    x = S.activations(300, 4096, seed=7, tensor_id=2, device=DEV)
    ref = A.quantize_activation(x, refine=True, exclude_mask=wm)
    out = A.alloc_activation(300, 4096, refine=True, device=DEV)
    A.quantize_noalloc(x, out, refine=True, exclude_mask=wm)
    torch.cuda.synchronize()
    same(out, ref, "activation 300x4096")

    # 3: smaller again - one decode token (the one-launch path), fp32
    say("case: noalloc activation 1x4096 fp32, refined")
    x1 = S.activations(1, 4096, seed=7, tensor_id=4, dtype=torch.float32, device=DEV)
    ref = A.quantize_activation(x1, refine=True, exclude_mask=wm)
    out = A.alloc_activation(1, 4096, refine=True, device=DEV)
    A.quantize_noalloc(x1, out, refine=True, exclude_mask=wm)
    torch.cuda.synchronize()
    same(out, ref, "activation 1x4096")

    # repeated calls into the same buffers give the same bytes
    A.quantize_noalloc(x1, out, refine=True, exclude_mask=wm)
    torch.cuda.synchronize()
    same(out, ref, "activation 1x4096, second call")


def test_noalloc_quantize_rejects_sizes_beyond_its_scratch():
    say("case: noalloc size limit")
    k_ok, k_bad = 491488, 491504
    x = torch.zeros(1, k_bad, dtype=torch.bfloat16, device=DEV)
    out = A.alloc_activation(1, k_bad, refine=False, device=DEV)
    with pytest.raises(A.AutofpError) as e:
        A.quantize_noalloc(x, out)
    assert e.value.status == 5
    x = S.activations(1, k_ok, seed=8, tensor_id=1, device=DEV)
    out = A.alloc_activation(1, k_ok, refine=False, device=DEV)
    A.quantize_noalloc(x, out)
    ref = A.quantize_activation(x)
    torch.cuda.synchronize()
    same(out, ref, "activation 1x491488")
