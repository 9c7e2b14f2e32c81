"""GPU parity of the device-side runtime policy (decisions must be identical
to the oracle's on the same signal values)."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import runtime_mixed_precision_amd as A

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(phase, la_steps, g_steps, batch):
    """la_steps: [steps][layers][batch] float32; returns levels [steps][batch][layers]."""
    state = A.policy_state(batch, DEV)
    out = []
    for s, la_layers in enumerate(la_steps):
        first = 6 if phase == 0 else 4
        levels = [[first] for _ in range(batch)]
        g = None if g_steps is None else torch.tensor(g_steps[s], dtype=torch.float32, device=DEV)
        for layer, la in enumerate(la_layers):
            la_t = torch.tensor(la, dtype=torch.float32, device=DEV)
            rows, lay = A.policy_update(phase, layer, la_t, state, g_e=g, new_sequence=(s == 0))
            r = rows.cpu().numpy()
            assert int(lay.cpu()[0]) == int(r.max())
            if layer + 1 < len(la_layers):
                for b in range(batch):
                    levels[b].append(int(r[b]))
        out.append(levels)
    return out


def test_prefill_policy_matches_oracle():
    say("case: prefill policy")
    rng = np.random.default_rng(0)
    batch, L = 6, 32
    la = rng.lognormal(-1.0, 0.3, (L, batch)).astype(np.float32)
    for b in range(batch):
        la[2 + b, b] *= 12.0                  # a spike at a different early layer per row
    la[:, 5] = np.linspace(1.0, 0.2, L)       # no spike: stays at 6
    got = run_gpu(0, [la.tolist()], None, batch)[0]
    for b in range(batch):
        want = O.policy_prefill(la[:, b].astype(np.float64).tolist())
        assert got[b] == want, (b, got[b], want)


def test_decode_policy_matches_oracle_over_steps():
    say("case: decode policy, 6 steps")
    rng = np.random.default_rng(1)
    batch, L, steps = 5, 32, 6
    la = rng.lognormal(-2.0, 0.5, (steps, L, batch)).astype(np.float32)
    la[:, 10:14, :] *= 3.0                    # sustained rise
    g = rng.uniform(0.0, 0.3, (steps, batch)).astype(np.float32)
    g[:, 0] = 0.05                            # row 0 always low entropy
    g[:, 1] = 0.5                             # row 1 always high entropy
    got = run_gpu(1, la.tolist(), g.tolist(), batch)
    for b in range(batch):
        st = O.PolicyState()
        for s in range(steps):
            want = O.policy_decode_step(la[s, :, b].astype(np.float64).tolist(), float(g[s, b]), st)
            assert got[s][b] == want, (s, b, got[s][b], want)
    levels = {v for s in got for row in s for v in row}
    assert levels == {2, 4, 6}                # the case exercises every level


@pytest.mark.parametrize("batch", [1, 3, 4, 5, 17])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_policy_layer_equals_signals_then_update(batch, dtype):
    """autofp_policy_layer (L_A and the policy step in one call: one launch up
    to 4 rows, two above) gives the same L_A, levels and state, value for
    value, as autofp_policy_signals followed by autofp_policy_update, over a
    prefill pass and decode steps."""
    say(f"case: policy_layer batch {batch} {dtype}")
    g = torch.Generator(device="cpu").manual_seed(batch)
    hidden = 4096
    st_a = A.policy_state(batch, DEV)
    st_b = A.policy_state(batch, DEV)
    for step, phase in enumerate((0, 1, 1)):
        g_e = None if phase == 0 else torch.rand(batch, generator=g).to(DEV) * 0.3
        h = torch.randn(batch, hidden, generator=g).to(DEV, dtype)
        for layer in range(12):
            scale = 0.05 + 0.2 * float(torch.rand(1, generator=g))
            h2 = (h.float() + scale * torch.randn(batch, hidden, generator=g).to(DEV)).to(dtype)
            la_b = A.policy_signals(h_prev=h, h_cur=h2)[1]
            rows_b, lay_b = A.policy_update(phase, layer, la_b, st_b, g_e=g_e, new_sequence=(step == 0))
            la_a, rows_a, lay_a = A.policy_layer(phase, layer, h, h2, st_a, g_e=g_e, new_sequence=(step == 0))
            assert torch.equal(la_a, la_b), (step, layer)
            assert torch.equal(rows_a, rows_b) and torch.equal(lay_a, lay_b), (step, layer)
            h = h2
        torch.cuda.synchronize()
        assert torch.equal(st_a.view(torch.uint8), st_b.view(torch.uint8)), step
