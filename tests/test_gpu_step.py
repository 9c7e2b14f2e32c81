"""A multi-layer decode step driven by the device-side policy, end to end on
the GPU (the 32-layer step with per-layer levels, at reduced width so the
parity checks stay cheap):

  G_E of the step's logits; per layer: encode the input, a = Wqkv x,
  o = Wo a[:, :H], h1 = h + o, [g|u] = Wgu h1, f = silu(g) * u,
  h2 = h1 + Wdown f, L_A(h, h2), policy update -> level of the next layer,
  read by the next layer's GEMVs on the device (no host round trip).

Checks, at batch 1, 16 and 64 over two steps:
  - the whole step captured in one HIP graph and replayed gives the same
    hidden states and levels as the eager run (bit for bit);
  - layer 0 runs at 4 bits, every level is in {2, 4, 6}, and a batched layer
    runs at the highest level of its rows (the policy's decisions themselves
    are checked against the oracle in test_gpu_policy.py);
  - the GEMVs of a layer match the oracle product (encoded by the oracle from
    the same float inputs) at the level the device chose.
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
H, F, V, LAYERS, STEPS = 512, 1024, 1000, 8, 2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Model:
    def __init__(self, batch):
        self.b = batch
        self.w, self.wqkv_f = [], []
        for layer in range(LAYERS):
            ws = {}
            for j, (name, n, k) in enumerate((("qkv", 3 * H, H), ("o", H, H), ("gu", 2 * F, H), ("down", H, F))):
                wf = S.weights(n, k, seed=40 + layer, tensor_id=j, device=DEV)
                ws[name] = A.quantize_weight(wf, refine=True)
                if name == "qkv":
                    self.wqkv_f.append(wf.cpu().numpy())
            self.w.append(ws)
        self.h0 = S.hidden(batch, H, seed=41, tensor_id=0, dtype=torch.float32, device=DEV)
        self.logits = [S.logits(batch, V, seed=42 + s, device=DEV) for s in range(STEPS)]
        # preallocated buffers: the step allocates nothing, so it can be captured
        self.xh = A.alloc_activation(batch, H, refine=True, device=DEV)
        self.xa = A.alloc_activation(batch, H, refine=True, device=DEV)
        self.xf = A.alloc_activation(batch, F, refine=True, device=DEV)
        self.qws = {k: torch.empty(A.workspace_bytes(0, batch, k), dtype=torch.uint8, device=DEV) for k in (H, F)}
        self.gws = {k: torch.empty(A.workspace_bytes(2, batch, k), dtype=torch.uint8, device=DEV) for k in (H, F)}
        self.sws = torch.empty(A.workspace_bytes(4, batch, V), dtype=torch.uint8, device=DEV)
        self.y = {"qkv": torch.empty(batch, 3 * H, device=DEV), "o": torch.empty(batch, H, device=DEV),
                  "gu": torch.empty(batch, 2 * F, device=DEV), "down": torch.empty(batch, H, device=DEV)}
        self.h = torch.empty(batch, H, device=DEV)
        self.h1 = torch.empty(batch, H, device=DEV)
        self.h2 = torch.empty(batch, H, device=DEV)
        self.a = torch.empty(batch, H, device=DEV)
        self.f = torch.empty(batch, F, device=DEV)
        self.g_e = torch.empty(batch, device=DEV)
        self.l_a = torch.empty(LAYERS, batch, device=DEV)
        self.rows = torch.empty(LAYERS, batch, dtype=torch.int32, device=DEV)
        self.lay = torch.empty(LAYERS + 1, dtype=torch.int32, device=DEV)
        self.g_log = torch.empty(STEPS, batch, device=DEV)
        self.h_log = torch.empty(STEPS, batch, H, device=DEV)
        self.state = A.policy_state(batch, DEV)

    def linear(self, name, layer, x_packed, k, bits_dev):
        A.gemv(self.w[layer][name], x_packed, bits_dev=bits_dev, out=self.y[name], workspace=self.gws[k])

    def step(self, s, record):
        A.policy_signals(logits=self.logits[s], out_entropy=self.g_e, workspace=self.sws)
        self.h.copy_(self.h0)
        self.lay[0].fill_(4)                          # decode steps start at 4 bits
        for layer in range(LAYERS):
            w = self.w[layer]
            bits = self.lay[layer:layer + 1]
            A.quantize_into(self.h, self.xh, refine=True, exclude_mask=w["qkv"].mask, workspace=self.qws[H])
            self.linear("qkv", layer, self.xh, H, bits)
            self.a.copy_(self.y["qkv"][:, :H])
            A.quantize_into(self.a, self.xa, refine=True, exclude_mask=w["o"].mask, workspace=self.qws[H])
            self.linear("o", layer, self.xa, H, bits)
            torch.add(self.h, self.y["o"], out=self.h1)
            A.quantize_into(self.h1, self.xh, refine=True, exclude_mask=w["gu"].mask, workspace=self.qws[H])
            self.linear("gu", layer, self.xh, H, bits)
            torch.mul(torch.nn.functional.silu(self.y["gu"][:, :F]), self.y["gu"][:, F:], out=self.f)
            A.quantize_into(self.f, self.xf, refine=True, exclude_mask=w["down"].mask, workspace=self.qws[F])
            self.linear("down", layer, self.xf, F, bits)
            torch.add(self.h1, self.y["down"], out=self.h2)
            A.policy_signals(h_prev=self.h, h_cur=self.h2, out_update=self.l_a[layer])
            A.policy_update(1, layer, self.l_a[layer], self.state, g_e=self.g_e,
                            new_sequence=(s == 0 and layer == 0), bits_rows=self.rows[layer],
                            bits_layer=self.lay[layer + 1:layer + 2])
            self.h.copy_(self.h2)
        if record:
            self.g_log[s].copy_(self.g_e)
            self.h_log[s].copy_(self.h)


def run(model, graph):
    """Both steps; returns host copies of (h per step, levels, rows, L_A, G_E)."""
    model.state.zero_()
    out = []
    for s in range(STEPS):
        if graph:
            g = torch.cuda.CUDAGraph()
            model.step(s, False)                      # warm-up outside the capture
            torch.cuda.synchronize()
            model.state.zero_() if s == 0 else None
            if s > 0:
                model.state.copy_(state_after[s - 1])
            with torch.cuda.graph(g):
                model.step(s, True)
            g.replay()
        else:
            model.step(s, True)
        torch.cuda.synchronize()
        out.append((model.h_log[s].cpu().clone(), model.lay.cpu().clone(), model.rows.cpu().clone(),
                    model.l_a.cpu().clone(), model.g_log[s].cpu().clone()))
        if not graph:
            state_after.append(model.state.clone())
    return out


state_after = []


@pytest.mark.parametrize("batch", [1, 16, 64])
def test_policy_driven_decode_step(batch):
    say(f"case: {LAYERS}-layer decode step with device policy, batch {batch}")
    state_after.clear()
    m = Model(batch)
    eager = run(m, graph=False)
    graphed = run(m, graph=True)
    levels_seen = set()
    for s in range(STEPS):
        he, lay_e, rows_e, la_e, g_e = eager[s]
        hg, lay_g, rows_g, la_g, g_g = graphed[s]
        assert torch.equal(he, hg), f"graph replay differs from the eager step (step {s})"
        assert torch.equal(lay_e, lay_g) and torch.equal(rows_e, rows_g)
        assert torch.equal(la_e, la_g) and torch.equal(g_e, g_g)
        assert torch.isfinite(he).all() and torch.isfinite(la_e).all()
        assert int(lay_e[0]) == 4
        assert set(rows_e.flatten().tolist()) <= {2, 4, 6}
        # a batched layer runs at the highest level of its rows
        assert lay_e[1:].tolist() == rows_e.max(dim=1).values.tolist()
        levels_seen |= set(lay_e.tolist())
    say(f"levels used: {sorted(levels_seen)}")


def test_step_layer_matches_oracle_at_device_level():
    """One layer of the step: the Wqkv GEMV at the level the device policy
    chose equals the oracle product at that level."""
    say("case: step layer vs oracle")
    batch = 4
    m = Model(batch)
    m.state.zero_()
    m.step(0, True)
    torch.cuda.synchronize()
    lay = m.lay.cpu().tolist()
    for layer, level in ((1, lay[1]), (LAYERS - 1, lay[LAYERS - 1])):
        w = m.w[layer]["qkv"]
        x = S.hidden(batch, H, seed=7, tensor_id=layer, dtype=torch.float32, device=DEV)
        xp = A.quantize_activation(x, refine=True, exclude_mask=w.mask)
        y = A.gemv(w, xp, bits_dev=m.lay[layer:layer + 1]).cpu().numpy()
        wn = m.wqkv_f[layer]
        bits, _ = O.select_weight_mask(wn, 0.2)
        wq = O.quantize_weight(wn, O.pack_nibbles(bits))
        xn = x.cpu().numpy()
        xq = O.quantize_activation(xn, refine=True, exclude_mask=wq["mask"]) if level == 6 else \
            O.quantize_activation(xn)
        ref = O.linear(wq, xq, level)
        err = np.abs(y - ref) / np.maximum(np.abs(ref), 0.01 * np.sqrt((ref ** 2).mean(axis=1, keepdims=True)))
        assert err.max() <= 1e-3, (layer, level, err.max())
