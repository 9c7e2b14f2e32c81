"""GPU parity of the runtime-policy signals G_E and L_A (tolerance 1e-3
relative, 1e-6 absolute, against the fp64 oracle)."""

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


def close(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert (np.abs(a - b) <= 1e-3 * np.abs(b) + 1e-6).all(), (a, b)


@pytest.mark.parametrize("batch,vocab", [(1, S.VOCAB), (4, S.VOCAB), (64, S.VOCAB), (3, 1000), (2, 37), (5, 130),
                                         (2, 8192), (2, 8195), (1, 4097)])
@pytest.mark.parametrize("top_k", [10, 1, 32, None])
def test_entropy(batch, vocab, top_k):
    k = vocab if top_k is None else top_k
    say(f"case: entropy B={batch} V={vocab} k={k}")
    z = S.logits(batch, vocab, seed=batch + vocab, device=DEV)
    g, _ = A.policy_signals(logits=z, params=A.default_params(top_k=k))
    close(g.cpu().numpy(), O.topk_entropy(z.cpu().numpy(), k))


def test_entropy_ties_and_extremes():
    say("case: entropy ties / extremes")
    V = 5000
    z = torch.full((3, V), -30.0, device=DEV)
    z[0, 100:110] = 2.0                       # ten equal leaders -> 1
    z[1, 7] = 80.0                            # one dominant logit -> 0
    z[2, ::400] = 5.0                         # 13 tied maxima: top-10 are all 5.0
    g, _ = A.policy_signals(logits=z)
    close(g.cpu().numpy(), O.topk_entropy(z.cpu().numpy(), 10))
    assert abs(float(g[0]) - 1.0) < 1e-6 and float(g[1]) < 1e-6


@pytest.mark.parametrize("top_k", [10, 32, None])
def test_entropy_masked_logits(top_k):
    """Vocabulary entries masked with -inf (probability 0): a row with fewer
    finite logits than top_k, one with a single finite logit, and one with the
    finite logits spread over many slices. G_E stays finite and equals the
    oracle's, which drops zero-probability terms."""
    V = S.VOCAB
    k = V if top_k is None else top_k
    say(f"case: entropy with -inf masked logits k={k}")
    z = torch.full((4, V), float("-inf"), device=DEV)
    z[0, [5, 900, 70000, V - 1]] = torch.tensor([1.0, 2.0, 0.5, 1.5], device=DEV)   # 4 finite
    z[1, 12345] = 3.0                                                                # 1 finite
    z[2, ::37] = S.logits(1, V, seed=5, device=DEV)[0, ::37]                        # 3467 finite
    z[3] = S.logits(1, V, seed=6, device=DEV)[0]
    z[3, 1000:50000] = float("-inf")
    g, _ = A.policy_signals(logits=z, params=A.default_params(top_k=k))
    gn = g.cpu().numpy()
    assert np.isfinite(gn).all(), gn
    close(gn, O.topk_entropy(z.cpu().numpy(), k))
    assert abs(float(gn[1])) < 1e-6


@pytest.mark.parametrize("top_k", [10, 32])
def test_entropy_leaders_in_one_place(top_k):
    """All leaders in the 16 logits one thread reads, or in the last, partial slice."""
    say(f"case: entropy concentrated leaders k={top_k}")
    V = S.VOCAB
    z = S.logits(3, V, seed=11, device=DEV)
    one_thread = [4 * 5 + i + 1024 * j for j in range(4) for i in range(4)]   # thread 5 of slice 0
    z[0, one_thread] = 40.0 + torch.arange(16, device=DEV, dtype=torch.float32) * 0.25
    z[1, V - 40:] = 30.0 + torch.arange(40, device=DEV, dtype=torch.float32) * 0.1
    z[2, 4096 * 7 + 64 * 3: 4096 * 7 + 64 * 3 + 40] = 25.0                    # one wavefront's range, tied
    g, _ = A.policy_signals(logits=z, params=A.default_params(top_k=top_k))
    close(g.cpu().numpy(), O.topk_entropy(z.cpu().numpy(), top_k))


def test_entropy_workspace_reuse():
    say("case: entropy workspace reused across shapes")
    ws = torch.empty(A.workspace_bytes(4, 8, S.VOCAB), dtype=torch.uint8, device=DEV)
    for b, v in ((8, S.VOCAB), (2, 5000), (8, S.VOCAB)):
        z = S.logits(b, v, seed=b * v, device=DEV)
        g, _ = A.policy_signals(logits=z, workspace=ws)
        close(g.cpu().numpy(), O.topk_entropy(z.cpu().numpy(), 10))


def test_update_norm_unaligned_rows():
    say("case: L_A on views that are not 16-byte aligned")
    base = S.hidden(4, 4097, seed=5, tensor_id=0, device=DEV)
    hp = base[:, 1:]                                   # row stride 4097, offset 1 element
    hc = (hp + 0.2).contiguous()[:, :]
    hp2 = torch.empty(4 * 4096 + 1, device=DEV)[1:].view(4, 4096)
    hp2.copy_(hp)
    _, la = A.policy_signals(h_prev=hp2, h_cur=hc)
    close(la.cpu().numpy(), O.update_norm(hp2.cpu().numpy(), hc.cpu().numpy(), 1e-6))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("batch,hidden", [(1, 4096), (16, 4096), (64, 4096), (3, 100)])
def test_update_norm(dtype, batch, hidden):
    say(f"case: L_A B={batch} H={hidden} {dtype}")
    hp = S.hidden(batch, hidden, seed=1, tensor_id=0, dtype=dtype, device=DEV)
    d = S.hidden(batch, hidden, seed=1, tensor_id=1, dtype=torch.float32, device=DEV)
    hc = (hp.float() + 0.1 * d).to(dtype)
    _, la = A.policy_signals(h_prev=hp, h_cur=hc)
    close(la.cpu().numpy(), O.update_norm(hp.float().cpu().numpy(), hc.float().cpu().numpy(), 1e-6))


def test_both_signals_in_one_call():
    say("case: both signals")
    z = S.logits(8, S.VOCAB, seed=3, device=DEV)
    hp = S.hidden(8, 4096, seed=3, tensor_id=0, device=DEV)
    hc = S.hidden(8, 4096, seed=3, tensor_id=1, device=DEV)
    g, la = A.policy_signals(logits=z, h_prev=hp, h_cur=hc)
    close(g.cpu().numpy(), O.topk_entropy(z.cpu().numpy(), 10))
    close(la.cpu().numpy(), O.update_norm(hp.cpu().numpy(), hc.cpu().numpy(), 1e-6))
