#!/usr/bin/env python3
"""AutoFP decode-step benchmark on one MI355X.

Workload: the decode hot path over Llama-3-8B-shaped layers
(Wqkv 6144x4096, Wo 4096x4096, Wgate|Wup fused 28672x4096, Wdown 4096x14336),
batch 1 by default, synthetic seeded data. One step =
  G_E of the next-token logits (128256 wide)                 (signal)
  three layers, at levels 2, 4 and 6, each:
    AutoFP GEMV against the packed weight, four per layer
    each output turned into the next input by one producer-epilogue call
    (copy / residual add + RMSNorm / SwiGLU, then the AutoFP encode); the
    layer's last one also takes L_A and the device-side policy update
Layers rotate through a pool larger than the 256 MB Infinity Cache, so the
weights stream from HBM. Everything is captured once per pool position in a
HIP graph and replayed.

Printed (stdout, one JSON line): whole-step algorithmic HBM GB/s, the GEMV
roofline (bytes / launch duration, HIP events around back-to-back GEMV-only
graphs), the prefill GEMM TFLOP/s, batched-decode and 32-layer-step lines,
decode attention over an AutoFP KV cache (16 x 32768 tokens, GQA 32/8), and
the CPU oracle on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_b1_pmc_traffic.md")
GEMV_SOURCES = ("runtime_mixed_precision_amd/csrc/gemv.hip", "runtime_mixed_precision_amd/csrc/afp_device.h",
                "runtime_mixed_precision_amd/csrc/afp_launch.h", "runtime_mixed_precision_amd/csrc/afp_act.h")
PEAK_FP16_TFLOPS = 2500.0      # dense fp16/bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0      # dense fp4/fp6 MFMA
LEVELS = (2, 4, 6)
SHAPES = (("wqkv", 6144, 4096), ("wo", 4096, 4096), ("wgateup", 28672, 4096), ("wdown", 4096, 14336))
METRIC = "AutoFP decode GEMV HBM GB/s (% peak); prefill GEMM TFLOP/s (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w_bytes(wp, level):
    b = wp.codes.numel() + wp.scales.numel() + 4
    if level == 6:
        b += wp.mask.numel() + wp.offsets.numel()
    return b


def x_bytes(rows, k, level):
    b = rows * (k // 2) + rows * (k // 16) + 4
    if level == 6:
        b += rows * ((k + 31) // 32) + rows * (k // 4)
    return b


def gemv_bytes(wp, b, level):
    """Algorithmic bytes of one GEMV: packed weight + packed activation + fp32 output."""
    return w_bytes(wp, level) + x_bytes(b, wp.k, level) + 4 * b * wp.rows


def encode_bytes(b, k, level):
    """bf16 input read + packed activation written."""
    return 2 * b * k + x_bytes(b, k, level)


def gemv_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per GEMV launch from the committed counter summary, or None
    when there is none or the GEMV sources changed since it was taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if "=" in line and line.strip().startswith(("traffic_bytes_per_launch", "gemv_source_sha256")):
            k, v = line.strip().strip("`").split("=", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("gemv_source_sha256") != gemv_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def pmc_pass(A, S, device):
    """Workload of the counter runs: each of the 12 batch-1 GEMV launches of
    the roofline (4 shapes x levels 2/4/6) three times, eagerly, then a plain
    64 MiB device copy whose FETCH_SIZE / WRITE_SIZE readings calibrate the
    counters."""
    import torch
    pool = build_pool(A, S, 3, device)
    bench = DecodeBench(A, S, pool, 1, device)
    torch.cuda.synchronize()
    for _ in range(3):
        bench.gemv_only(0)
    torch.cuda.synchronize()
    src = torch.ones(64 << 18, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("pmc pass done: 36 GEMV launches, one 64 MiB copy")


def pmc_batch_pass(A, S, device):
    """Workload of the batched-decode counter runs: the 12 GEMV launches at
    64 tokens (4 shapes x levels 2/4/6) and the 28672 x 8192 projection at 64
    tokens, level 4, three times each, eagerly, then the 64 MiB copy that
    calibrates the traffic counters."""
    import torch
    pool = build_pool(A, S, 3, device)
    bench = DecodeBench(A, S, pool, 64, device)
    n, k = 28672, 8192
    w70 = A.quantize_weight(S.weights(n, k, seed=700, tensor_id=0, device=device))
    x70 = A.quantize_activation(S.activations(64, k, seed=700, tensor_id=1, outlier_frac=0.0, device=device))
    y70 = torch.empty(64, n, dtype=torch.float32, device=device)
    ws70 = torch.empty(A.workspace_bytes(2, 64, k), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    for _ in range(3):
        bench.gemv_only(0)
        A.gemv(w70, x70, bits=4, out=y70, workspace=ws70)
    torch.cuda.synchronize()
    src = torch.ones(64 << 18, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("pmc batch pass done: 3 x (12 GEMV launches at 64 tokens + the 70B projection), one 64 MiB copy")


def pmc_prefill_pass(A, S, device):
    """Workload of the prefill counter runs: the GEMMs of 2048 tokens against
    Wup (14336 x 4096) and Wdown (4096 x 14336) at levels 4 and 6, three
    times each, eagerly, then the 64 MiB copy that calibrates the traffic
    counters."""
    import torch
    M = 2048
    for name, n, k, tid in (("wup", 14336, 4096, 1), ("wdown", 4096, 14336, 3)):
        w = S.weights(n, k, seed=200, tensor_id=tid, device=device)
        wp = A.quantize_weight(w, refine=True)
        del w
        x = S.activations(M, k, seed=200, tensor_id=10 + tid, outlier_frac=0.005, outlier_scale=30.0,
                          device=device)
        ws = torch.empty(A.workspace_bytes(3, M, k), dtype=torch.uint8, device=device)
        y = torch.empty(M, n, dtype=torch.bfloat16, device=device)
        for level in (4, 6):
            xp = A.quantize_activation(x, refine=(level == 6), exclude_mask=wp.mask if level == 6 else None)
            torch.cuda.synchronize()
            for _ in range(3):
                A.gemm(wp, xp, bits=level, out=y, workspace=ws)
            torch.cuda.synchronize()
        del wp, x, ws, y
    src = torch.ones(64 << 18, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("pmc prefill pass done: 3 x (Wup, Wdown) x levels 4, 6 at 2048 tokens, one 64 MiB copy")


def build_pool(A, S, n_layers, device):
    pool = []
    for i in range(n_layers):
        layer = {}
        for j, (name, n, k) in enumerate(SHAPES):
            w = S.weights(n, k, seed=100 + i, tensor_id=j, device=device)
            layer[name] = A.quantize_weight(w, refine=True)
            del w
        pool.append(layer)
        log(f"packed layer {i + 1}/{n_layers}")
    import torch
    torch.cuda.synchronize()
    return pool


class DecodeBench:
    def __init__(self, A, S, pool, batch, device):
        import torch
        self.A, self.pool, self.b, self.device = A, pool, batch, device
        self.p = A.default_params()
        self.x_in = {name: S.activations(batch, k, seed=7, tensor_id=j, outlier_frac=0.0, device=device)
                     for j, (name, n, k) in enumerate(SHAPES)}
        self.xq = {name: A.alloc_activation(batch, k, refine=True, device=device) for name, n, k in SHAPES}
        self.y = {name: torch.empty(batch, n, dtype=torch.float32, device=device) for name, n, k in SHAPES}
        ks = sorted({k for _, _, k in SHAPES})
        # encode / epilogue workspaces (AUTOFP_OP_EPILOGUE: the encode's plus the RMSNorm row scales)
        self.qws = {k: torch.empty(A.workspace_bytes(8, batch, k), dtype=torch.uint8, device=device) for k in ks}
        self.gws = {k: torch.empty(A.workspace_bytes(2, batch, k), dtype=torch.uint8, device=device) for k in ks}
        self.logits = S.logits(batch, S.VOCAB, seed=7, device=device)
        self.sws = torch.empty(A.workspace_bytes(4, batch, S.VOCAB), dtype=torch.uint8, device=device)
        self.h_prev = S.hidden(batch, S.HIDDEN, seed=7, tensor_id=0, device=device)
        self.h_cur = (self.h_prev + 0.05 * S.hidden(batch, S.HIDDEN, seed=7, tensor_id=1, device=device)).contiguous()
        self.g_e = torch.zeros(batch, dtype=torch.float32, device=device)
        self.l_a = torch.zeros(batch, dtype=torch.float32, device=device)
        self.state = A.policy_state(batch, device)
        self.bits_rows = torch.zeros(batch, dtype=torch.int32, device=device)
        self.bits_layer = torch.zeros(1, dtype=torch.int32, device=device)
        self._chain_buffers(S)
        # activations encoded once per level for the GEMV-only timing
        self.xq_l = {}
        for name, n, k in SHAPES:
            for level in LEVELS:
                wp = pool[0][name]
                self.xq_l[(name, level)] = A.quantize_activation(
                    self.x_in[name], refine=(level == 6), exclude_mask=wp.mask if level == 6 else None)

    def layers_of(self, s):
        P = len(self.pool)
        return [self.pool[(len(LEVELS) * s + j) % P] for j in range(len(LEVELS))]

    def _chain_buffers(self, S):
        """Buffers of the chained step: the hidden state (ping-pong), the
        linear outputs z, the encoded input of each linear."""
        import torch
        if hasattr(self, "z"):
            return
        A, b, dev = self.A, self.b, self.device
        H = S.HIDDEN
        self.h0 = S.hidden(b, H, seed=7, tensor_id=0, device=dev)
        self.hbuf = [torch.empty(b, H, device=dev) for _ in range(2)]
        self.h1 = torch.empty(b, H, device=dev)
        self.z = {name: torch.empty(b, n, dtype=torch.float32, device=dev) for name, n, k in SHAPES}
        self.f = torch.empty(b, S.FFN, device=dev)
        self.a = torch.empty(b, H, device=dev)
        self.nrm = torch.empty(b, H, device=dev)

    def step(self, s):
        """One decode step with the layers chained and each linear's output
        post-processed into the next linear's input in one call
        (autofp_epilogue_quantize: copy / residual add + RMSNorm / SwiGLU,
        then the encode): G_E, then per layer GEMV Wqkv -> copy of the first
        4096 outputs -> GEMV Wo -> h1 = h + o, RMSNorm(h1) encoded -> GEMV
        Wgate|Wup -> silu(g) * u -> GEMV Wdown -> h2 = h1 + d, RMSNorm(h2)
        encoded for the next layer, with L_A(h, h2) and the policy update in
        the same call (autofp_layer_epilogue)."""
        A, p = self.A, self.p
        A.policy_signals(logits=self.logits, out_entropy=self.g_e, params=p, workspace=self.sws)
        layers = self.layers_of(s)
        h_in = self.h0
        A.quantize_into(h_in, self.xq["wqkv"], refine=True, exclude_mask=layers[0]["wqkv"].mask,
                        workspace=self.qws[4096], params=p)
        for j, (layer, level) in enumerate(zip(layers, LEVELS)):
            h_out = self.hbuf[j % 2]
            nxt = layers[j + 1] if j + 1 < len(layers) else layers[0]
            g = lambda name, k: A.gemv(layer[name], self.xq[name], bits=level, out=self.z[name],
                                       workspace=self.gws[k], params=p)
            g("wqkv", 4096)
            A.epilogue_quantize("copy", self.z["wqkv"], self.xq["wo"], refine=True, exclude_mask=layer["wo"].mask,
                                workspace=self.qws[4096], params=p)
            g("wo", 4096)
            A.epilogue_quantize("residual_rmsnorm", self.z["wo"], self.xq["wgateup"], residual=h_in, v_out=self.h1,
                                refine=True, exclude_mask=layer["wgateup"].mask, workspace=self.qws[4096], params=p)
            g("wgateup", 4096)
            A.epilogue_quantize("swiglu", self.z["wgateup"], self.xq["wdown"], refine=True,
                                exclude_mask=layer["wdown"].mask, workspace=self.qws[14336], params=p)
            g("wdown", 14336)
            A.layer_epilogue(self.z["wdown"], self.xq["wqkv"], self.h1, h_out, h_in, 1, j, self.state, g_e=self.g_e,
                             l_a=self.l_a, bits_rows=self.bits_rows, bits_layer=self.bits_layer, refine=True,
                             exclude_mask=nxt["wqkv"].mask, workspace=self.qws[4096], params=p)
            h_in = h_out

    def step_unfused(self, s):
        """The same chained step with the elementwise steps as separate torch
        kernels and a separate encode launch per linear input (no producer
        epilogue): the comparison for the fused form."""
        import torch
        A, p = self.A, self.p
        A.policy_signals(logits=self.logits, out_entropy=self.g_e, params=p, workspace=self.sws)
        layers = self.layers_of(s)
        h_in = self.h0
        A.quantize_into(h_in, self.xq["wqkv"], refine=True, exclude_mask=layers[0]["wqkv"].mask,
                        workspace=self.qws[4096], params=p)
        for j, (layer, level) in enumerate(zip(layers, LEVELS)):
            h_out = self.hbuf[j % 2]
            nxt = layers[j + 1] if j + 1 < len(layers) else layers[0]
            g = lambda name, k: A.gemv(layer[name], self.xq[name], bits=level, out=self.z[name],
                                       workspace=self.gws[k], params=p)
            g("wqkv", 4096)
            self.a.copy_(self.z["wqkv"][:, :4096])
            A.quantize_into(self.a, self.xq["wo"], refine=True, exclude_mask=layer["wo"].mask,
                            workspace=self.qws[4096], params=p)
            g("wo", 4096)
            torch.add(h_in, self.z["wo"], out=self.h1)
            rmsnorm_into(self.h1, self.nrm)
            A.quantize_into(self.nrm, self.xq["wgateup"], refine=True, exclude_mask=layer["wgateup"].mask,
                            workspace=self.qws[4096], params=p)
            g("wgateup", 4096)
            silu_mul(self.z["wgateup"], 14336, self.f)
            A.quantize_into(self.f, self.xq["wdown"], refine=True, exclude_mask=layer["wdown"].mask,
                            workspace=self.qws[14336], params=p)
            g("wdown", 14336)
            torch.add(self.h1, self.z["wdown"], out=h_out)
            rmsnorm_into(h_out, self.nrm)
            A.quantize_into(self.nrm, self.xq["wqkv"], refine=True, exclude_mask=nxt["wqkv"].mask,
                            workspace=self.qws[4096], params=p)
            A.policy_layer(1, j, h_in, h_out, self.state, g_e=self.g_e, l_a=self.l_a,
                           bits_rows=self.bits_rows, bits_layer=self.bits_layer, params=p)
            h_in = h_out

    def step_bytes(self):
        """Algorithmic bytes of the chained step: logits; the first encode (fp32
        hidden in, packed out); per layer the four GEMVs (packed weight at the
        layer's level, packed activation, fp32 output) and the four epilogues
        (fp32 inputs read: the copied 4096 outputs, residual + output, both
        SwiGLU halves; fp32 hidden states written by the residual steps;
        the refined packed activation written); L_A reads h and h2."""
        b, H, F = self.b, 4096, 14336
        tot = 4 * b * 128256 + 4 * b * H + x_bytes(b, H, 6)
        for layer, level in zip(self.layers_of(0), LEVELS):
            for name, n, k in SHAPES:
                tot += gemv_bytes(layer[name], b, level)
            tot += 4 * b * H + x_bytes(b, H, 6)                     # copy
            tot += 3 * 4 * b * H + x_bytes(b, H, 6)                 # residual (z, h read; h1 written)
            tot += 2 * 4 * b * F + x_bytes(b, F, 6)                 # SwiGLU
            tot += 3 * 4 * b * H + x_bytes(b, H, 6)                 # residual (z, h1 read; h2 written)
            tot += 2 * 4 * b * H                                    # L_A
        return tot

    def gemv_only(self, s):
        for layer, level in zip(self.layers_of(s), LEVELS):
            for name, n, k in SHAPES:
                self.A.gemv(layer[name], self.xq_l[(name, level)], bits=level, out=self.y[name],
                            workspace=self.gws[k], params=self.p)

    def gemv_only_bytes(self):
        tot = 0
        for layer, level in zip(self.layers_of(0), LEVELS):
            for name, n, k in SHAPES:
                tot += gemv_bytes(layer[name], self.b, level)
        return tot


class Step32:
    """The full decode step of a 32-layer Llama-3-8B-shaped model under the
    device-side policy: G_E of the step's logits, then per layer
    a = Wqkv RMSNorm(h) (first 4096 outputs as the attention stand-in),
    o = Wo a, h1 = h + o, [g|u] = Wgate|Wup RMSNorm(h1), f = silu(g) * u,
    h2 = h1 + Wdown f, each linear's output turned into the next linear's
    encoded input by one producer-epilogue call (the residual adds with the
    following RMSNorm, unit gain, so the hidden state stays finite over 32
    layers of random weights), the last with L_A(h, h2) and the policy update,
    whose level the next layer's GEMVs read on the device. Several consecutive steps
    (logits drawn per step) form one HIP graph; the levels chosen are logged
    on the device and read back after timing."""

    def __init__(self, A, S, layers, batch, device, steps=4):
        import torch
        self.A, self.S, self.layers, self.b, self.T = A, S, layers, batch, steps
        H, F, V = S.HIDDEN, S.FFN, S.VOCAB
        self.H, self.F, self.V = H, F, V
        L = len(layers)
        self.h0 = S.hidden(batch, H, seed=41, tensor_id=0, dtype=torch.float32, device=device)
        self.logits = [S.logits(batch, V, seed=42 + s, device=device) for s in range(steps)]
        # odd steps have one dominant next token (G_E near 0, below tau): the
        # low-entropy regime of the policy, where lower levels are reached
        for s in range(1, steps, 2):
            self.logits[s][:, 17] += 25.0
        self.xq = {name: A.alloc_activation(batch, k, refine=True, device=device) for name, n, k in SHAPES}
        self.qws = {k: torch.empty(A.workspace_bytes(8, batch, k), dtype=torch.uint8, device=device) for k in (H, F)}
        self.gws = {k: torch.empty(A.workspace_bytes(2, batch, k), dtype=torch.uint8, device=device) for k in (H, F)}
        self.sws = torch.empty(A.workspace_bytes(4, batch, V), dtype=torch.uint8, device=device)
        self.y = {"wqkv": torch.empty(batch, 3 * 2048, device=device), "wo": torch.empty(batch, H, device=device),
                  "wgateup": torch.empty(batch, 2 * F, device=device), "wdown": torch.empty(batch, H, device=device)}
        self.hb = [torch.empty(batch, H, device=device) for _ in range(2)]
        self.h1 = torch.empty(batch, H, device=device)
        self.g_e = torch.empty(batch, device=device)
        self.l_a = torch.empty(batch, device=device)
        self.rows = torch.empty(batch, dtype=torch.int32, device=device)
        self.lay = torch.empty(steps, L + 1, dtype=torch.int32, device=device)
        self.state = A.policy_state(batch, device)

    def run(self):
        A = self.A
        for s in range(self.T):
            lay = self.lay[s]
            A.policy_signals(logits=self.logits[s], out_entropy=self.g_e, workspace=self.sws)
            lay[0].fill_(4)                                   # a decode step starts at 4 bits
            h_in = self.h0
            A.quantize_into(h_in, self.xq["wqkv"], refine=True, exclude_mask=self.layers[0]["wqkv"].mask,
                            workspace=self.qws[self.H])
            for i, w in enumerate(self.layers):
                bits = lay[i:i + 1]
                h_out = self.hb[i % 2]
                nxt = self.layers[(i + 1) % len(self.layers)]
                A.gemv(w["wqkv"], self.xq["wqkv"], bits_dev=bits, out=self.y["wqkv"], workspace=self.gws[self.H])
                A.epilogue_quantize("copy", self.y["wqkv"], self.xq["wo"], refine=True, exclude_mask=w["wo"].mask,
                                    workspace=self.qws[self.H])
                A.gemv(w["wo"], self.xq["wo"], bits_dev=bits, out=self.y["wo"], workspace=self.gws[self.H])
                A.epilogue_quantize("residual_rmsnorm", self.y["wo"], self.xq["wgateup"], residual=h_in,
                                    v_out=self.h1, refine=True, exclude_mask=w["wgateup"].mask,
                                    workspace=self.qws[self.H])
                A.gemv(w["wgateup"], self.xq["wgateup"], bits_dev=bits, out=self.y["wgateup"],
                       workspace=self.gws[self.H])
                A.epilogue_quantize("swiglu", self.y["wgateup"], self.xq["wdown"], refine=True,
                                    exclude_mask=w["wdown"].mask, workspace=self.qws[self.F])
                A.gemv(w["wdown"], self.xq["wdown"], bits_dev=bits, out=self.y["wdown"], workspace=self.gws[self.F])
                A.layer_epilogue(self.y["wdown"], self.xq["wqkv"], self.h1, h_out, h_in, 1, i, self.state,
                                 g_e=self.g_e, new_sequence=(s == 0 and i == 0), l_a=self.l_a, bits_rows=self.rows,
                                 bits_layer=lay[i + 1:i + 2], refine=True, exclude_mask=nxt["wqkv"].mask,
                                 workspace=self.qws[self.H])
                h_in = h_out

    def bytes_of(self, lay):
        """Algorithmic bytes of the logged steps: logits; per step the first
        encode; per layer the packed weights at the level the layer ran, its
        packed activations and fp32 outputs, the four producer epilogues (fp32
        reads and writes, the refined packed activation written) and the L_A
        reads."""
        b, H, F, tot = self.b, self.H, self.F, 0
        for s in range(self.T):
            tot += 4 * b * self.V + 4 * b * H + x_bytes(b, H, 6)
            for i, w in enumerate(self.layers):
                L = int(lay[s][i])
                for name, wp in w.items():
                    tot += gemv_bytes(wp, b, L)
                tot += 4 * b * H + 2 * (3 * 4 * b * H) + 2 * 4 * b * F
                tot += 3 * x_bytes(b, H, 6) + x_bytes(b, F, 6) + 2 * 4 * b * H
        return tot


def torch_add(x, y, out):
    import torch
    torch.add(x, y, out=out)


def rmsnorm_into(h, out):
    """RMSNorm with unit gain and eps 1e-5 in torch ops (the unfused step's
    counterpart of the residual_rmsnorm epilogue)."""
    import torch
    torch.mul(h, torch.rsqrt(h.pow(2).mean(dim=1, keepdim=True) + 1e-5), out=out)


def silu_mul(gu, F, out):
    import torch
    torch.mul(torch.nn.functional.silu(gu[:, :F]), gu[:, F:], out=out)


def step32_bench(A, S, device, batches=(1, 16, 64), reps=3):
    """C4: the 32-layer step at each batch size, four steps per graph."""
    import torch
    layers = []
    for i in range(32):
        layer = {}
        for j, (name, n, k) in enumerate(SHAPES):
            w = S.weights(n, k, seed=300 + i, tensor_id=j, device=device)
            layer[name] = A.quantize_weight(w, refine=True)
            del w
        layers.append(layer)
    torch.cuda.synchronize()
    log("packed 32 layers for the 32-layer step")
    out = {"workload": "32 Llama-3-8B-shaped layers (Wqkv, Wo, Wgate|Wup, Wdown; 128256-wide logits), "
                       "levels chosen per layer on the device (G_E + L_A policy), 4 steps per graph"}
    for b in batches:
        m = Step32(A, S, layers, b, device)
        m.state.zero_()
        m.run()                                   # eager pass: code objects, buffers
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        m.state.zero_()
        with torch.cuda.graph(g):
            m.run()
        g.replay()
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(reps):
            g.replay()
        en.record()
        torch.cuda.synchronize()
        ms = st.elapsed_time(en) / (reps * m.T)
        lay = m.lay.cpu().tolist()
        by = m.bytes_of(lay) / m.T
        mix = {str(L): sum(row[:32].count(L) for row in lay) for L in (2, 4, 6)}
        out[f"b{b}"] = {"ms_per_step": round(ms, 4), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                        "mb_per_step": round(by / 1e6, 1), "level_mix_layers": mix}
        log(f"32-layer step, batch {b}: {ms:.3f} ms, {by / (ms * 1e-3) / 1e9:.1f} GB/s, levels {mix}")
        del m, g
    del layers
    torch.cuda.empty_cache()
    return out


def capture(fn_list):
    import torch
    graphs = []
    for fn in fn_list:
        fn()                                   # eager pass: code objects loaded, buffers touched
    torch.cuda.synchronize()
    for fn in fn_list:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_graphs(graphs, reps, warmup):
    """Replay graphs round-robin; returns ms per replay (HIP events on the
    replay stream, synchronized on both sides)."""
    import torch
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def prefill_bench(A, S, device, reps):
    import torch
    out = {}
    M = 2048
    for name, n, k, tid in (("wup", 14336, 4096, 1), ("wdown", 4096, 14336, 3)):
        w = S.weights(n, k, seed=200, tensor_id=tid, device=device)
        wp = A.quantize_weight(w, refine=True)
        del w
        x = S.activations(M, k, seed=200, tensor_id=10 + tid, outlier_frac=0.005, outlier_scale=30.0,
                          device=device)
        ws = torch.empty(A.workspace_bytes(3, M, k), dtype=torch.uint8, device=device)
        y = torch.empty(M, n, dtype=torch.bfloat16, device=device)
        for level in (4, 6):
            xp = A.quantize_activation(x, refine=(level == 6), exclude_mask=wp.mask if level == 6 else None)
            fn = lambda: A.gemm(wp, xp, bits=level, out=y, workspace=ws)
            g = capture([fn])
            ms = time_graphs(g, reps, 2)
            tflops = 2.0 * M * n * k / (ms * 1e-3) / 1e12
            out[f"{name}_l{level}"] = {"ms": round(ms, 4), "tflops": round(tflops, 1)}
        del wp, x, ws, y
    vals = [v["tflops"] for v in out.values()]
    best4 = max(out["wup_l4"]["tflops"], out["wdown_l4"]["tflops"])
    best6 = max(out["wup_l6"]["tflops"], out["wdown_l6"]["tflops"])
    return {"workload": "X[2048x4096] (Wup 14336x4096) and X'[2048x14336] (Wdown 4096x14336), "
                        "bf16 out, levels 4 and 6",
            "per_gemm": out, "tflops_mean": round(sum(vals) / len(vals), 1),
            "frac_fp16_mfma_peak": round(best4 / PEAK_FP16_TFLOPS, 4),
            "frac_fp4_mfma_peak": round(best4 / PEAK_FP4_TFLOPS, 4),
            "frac_note": "fracs of the best 4-bit (level 4) GEMM; level 6: "
                         f"{best6 / PEAK_FP16_TFLOPS:.4f} of the fp16 peak"}


def formats_bench(A, S, device, reps=5, pool_n=6):
    """The format variants ([AE] §6.5 / Fig. 14(a) exponent-scaled offsets,
    App. I AutoFP8, App. B.2 FP6g) at their top level on the Wup shape
    (14336 x 4096): prefill GEMM TFLOP/s at 2048 tokens, one-token decode
    GB/s (all packed weight and activation bytes, weights rotated over a pool
    larger than the Infinity Cache), and stored bits per weight."""
    import torch
    n, k, M = 14336, 4096, 2048
    out = {}
    x = S.activations(M, k, seed=300, tensor_id=1, outlier_frac=0.005, outlier_scale=30.0, device=device)
    x1 = x[:1].contiguous()
    ws = torch.empty(A.workspace_bytes(3, M, k), dtype=torch.uint8, device=device)
    y = torch.empty(M, n, dtype=torch.bfloat16, device=device)
    y1 = torch.empty(1, n, dtype=torch.float32, device=device)
    for fmt, level in (("autofp6", 6), ("autofp6e", 6), ("autofp8", 6), ("autofp8", 8), ("fp6g", 6)):
        pool = []
        for i in range(pool_n):
            w = S.weights(n, k, seed=300 + i, tensor_id=0, device=device)
            pool.append(A.quantize_weight(w, format=fmt))
            del w
        wp = pool[0]
        refine = fmt != "fp6g"
        xp = A.quantize_activation(x, refine=refine, exclude_mask=wp.mask, format=fmt)
        xp1 = A.quantize_activation(x1, refine=refine, exclude_mask=wp.mask, format=fmt)
        ms = time_graphs(capture([lambda: A.gemm(wp, xp, bits=level, out=y, workspace=ws)]), reps, 2)
        g1 = capture([lambda w_=w_: A.gemv(w_, xp1, bits=level, out=y1, workspace=ws) for w_ in pool])
        us = time_graphs(g1, 20, 3) * 1e3
        by = wp.nbytes + xp1.nbytes + 4 * n
        out[f"{fmt}_l{level}"] = {"prefill_ms": round(ms, 4), "prefill_tflops": round(2.0 * M * n * k / (ms * 1e-3) / 1e12, 1),
                                  "decode_us": round(us, 2), "decode_gbs": round(by / (us * 1e-6) / 1e9, 1),
                                  "bits_per_weight": round(8.0 * wp.nbytes / (n * k), 3)}
        del pool, wp, xp, xp1, g1
    del x, x1, ws, y, y1
    return {"workload": "Wup 14336x4096: X[2048x4096] prefill (bf16 out) and one-token decode, each format at its top level",
            "per_format": out}


def gptq_bench(A, S, device, reps=3):
    """Refinement-aware GPTQ ([AE] App. E, Algorithm 1) on the Wo (4096 x 4096)
    and Wgate (14336 x 4096) shapes, calibration X of 2048 correlated tokens.
    The caller's preparation (H = X^T X, 1 % damping, U = the upper Cholesky
    factor of H^-1) runs in torch.linalg and is not timed. Algorithmic bytes
    of the propagation (the dominant kernel): per group j, the fp64 working
    weights of the later columns read and written (16 B each), U's 16 rows
    over them and the 16 fp64 errors per row."""
    import torch
    out = {}
    x = S.calibration(2048, 4096, seed=500, tensor_id=0).to(device=device, dtype=torch.float64)
    h = x.T @ x
    h = h + 0.01 * torch.mean(torch.diagonal(h)) * torch.eye(4096, dtype=torch.float64, device=device)
    u = torch.linalg.cholesky(torch.cholesky_inverse(torch.linalg.cholesky(h)), upper=True).contiguous()
    hd = torch.diagonal(h).contiguous()
    del x
    for name, n in (("wo", 4096), ("wgate", 14336)):
        k = 4096
        w = S.weights(n, k, seed=500, tensor_id=1, device=device)
        ws = torch.empty(A.workspace_bytes(7, n, k), dtype=torch.uint8, device=device)
        A.gptq_quantize(w, u, hd, workspace=ws)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            A.gptq_quantize(w, u, hd, workspace=ws)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        G = k // 16
        prop = sum(16 * n * (k - 16 * (j + 1)) + 8 * 16 * (k - 16 * (j + 1)) + 8 * 16 * n for j in range(G - 1))
        out[name] = {"ms": round(ms, 2), "groups": G, "launches": 4 * G,
                     "propagate_bytes": prop, "propagate_bytes_over_total_time_gbs": round(prop / (ms * 1e-3) / 1e9, 1)}
        del w, ws
    return {"workload": "GPTQ of W [n x 4096] (Wo n = 4096, Wgate n = 14336), 2048 calibration tokens", **out}


def gemv_70b(A, S, device, batch=64, pool_n=5):
    """The 70B-shaped projection (28672 x 8192) at 64 tokens, level 4: weights
    rotated over a pool larger than the Infinity Cache, one graph per weight."""
    import torch
    n, k = 28672, 8192
    pool = []
    for i in range(pool_n):
        w = S.weights(n, k, seed=700 + i, tensor_id=0, device=device)
        pool.append(A.quantize_weight(w))
        del w
    x = S.activations(batch, k, seed=700, tensor_id=1, outlier_frac=0.0, device=device)
    xp = A.quantize_activation(x)
    y = torch.empty(batch, n, dtype=torch.float32, device=device)
    ws = torch.empty(A.workspace_bytes(2, batch, k), dtype=torch.uint8, device=device)
    graphs = capture([lambda wp=wp: A.gemv(wp, xp, bits=4, out=y, workspace=ws) for wp in pool])
    ms = time_graphs(graphs, 20, 3)
    by = gemv_bytes(pool[0], batch, 4)
    out = {"workload": "W 28672x8192 at 64 tokens, level 4", "us": round(ms * 1e3, 2),
           "gbs": round(by / (ms * 1e-3) / 1e9, 1), "tflops": round(2.0 * batch * n * k / (ms * 1e-3) / 1e12, 1)}
    del pool, graphs
    return out


def kv_bench(A, S, device, batch=16, ctx=32768, h_q=32, h_kv=8, reps=20):
    """Decode attention over an AutoFP KV cache: ``batch`` sequences of ``ctx``
    tokens, h_q query / h_kv KV heads, head_dim 128, bf16 K/V/q. Two caches:
    every page a base page (the 4-bit configuration, level 4) and every token
    refined (level 6). Algorithmic bytes per launch: each cached token's codes
    and E4M3 scales (72 B per KV head, K and V; + 64 B of offsets per refined
    token at level 6), the page table, q (bf16) and the fp32 output."""
    import numpy as np
    import torch
    out = {"workload": f"{batch} sequences x {ctx} tokens, {h_q} query / {h_kv} KV heads, head_dim 128, "
                       "bf16 K/V/q; level 4 over base pages, level 6 over refined pages"}
    hd = 128
    for frac, level in ((0.0, 4), (1.0, 6)):
        plan = S.kv_page_plan([ctx] * batch, frac, seed=41)
        n = batch * ctx
        cache = A.KVCache(plan["n_pages"], h_kv, batch, plan["max_pages"], device=device)
        cache.page_kind.copy_(torch.from_numpy(plan["page_kind"]))
        cache.page_tokens.copy_(torch.from_numpy(plan["page_tokens"]))
        cache.page_table.copy_(torch.from_numpy(plan["page_table"]))
        cache.seq_pages.copy_(torch.from_numpy(plan["seq_pages"]))
        slots = torch.from_numpy(np.concatenate(plan["slots"])).to(device)
        k = S.kv_tokens(n, h_kv, seed=42, tensor_id=1, device=device)
        v = S.kv_tokens(n, h_kv, seed=42, tensor_id=2, device=device)
        A.kv_write(cache, k, v, slots, set_scale=True)
        del k, v, slots
        q = S.kv_tokens(batch, h_q, seed=43, tensor_id=3, device=device)
        y = torch.empty(batch, h_q, hd, dtype=torch.float32, device=device)
        ws = torch.empty(A.workspace_bytes(6, batch * h_q, plan["max_pages"]), dtype=torch.uint8, device=device)
        g = capture([lambda: A.kv_attention(q, cache, bits=level, out=y, workspace=ws)])
        ms = time_graphs(g, reps, 3)
        n_ref = int(sum(r.sum() for r in plan["refine"]))
        tok_bytes = 2 * h_kv * (72 * n + (64 * n_ref if level == 6 else 0))
        by = tok_bytes + 4 * batch * plan["max_pages"] + 2 * batch * h_q * hd + 4 * batch * h_q * hd
        gbs = by / (ms * 1e-3) / 1e9
        out[f"l{level}"] = {"us": round(ms * 1e3, 2), "bytes": int(by), "gbs": round(gbs, 1),
                            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "refined_tokens": n_ref}
        log(f"kv attention level {level}: {ms * 1e3:.1f} us, {by / 1e6:.1f} MB, {gbs:.1f} GB/s")
        del cache, q, y, ws, g
        torch.cuda.empty_cache()
    return out


def _cpu_worker(args):
    """One worker of the CPU baseline (a fresh interpreter): the oracle on its
    share of the sample, one BLAS thread, for ``target_s`` seconds."""
    batch, target_s, wid = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    from runtime_mixed_precision_amd import synthetic as S

    rows = 512
    with threadpool_limits(limits=1):
        prepared = []
        for j, (name, n, k) in enumerate(SHAPES):
            w = S.weights(rows, k, seed=300 + wid, tensor_id=j).numpy()
            x = S.activations(batch, k, seed=300 + wid, tensor_id=10 + j, outlier_frac=0.0).float().numpy()
            bits, _ = O.select_weight_mask(w, 0.2)
            wq = O.quantize_weight(w, O.pack_nibbles(bits))
            prepared.append((w, x, wq, k))
        done_bytes = 0
        passes = 0
        t0 = time.perf_counter()
        while True:
            for w, x, wq, k in prepared:
                for level in LEVELS:
                    xq = O.quantize_activation(x, refine=(level == 6),
                                               exclude_mask=wq["mask"] if level == 6 else None)
                    O.linear(wq, xq, level)
                    wb = wq["codes"].size + wq["scales"].size + 4
                    if level == 6:
                        wb += wq["mask"].size + wq["offsets"].size
                    done_bytes += wb + x_bytes(batch, k, level) + 4 * batch * rows + encode_bytes(batch, k, level)
            passes += 1
            if time.perf_counter() - t0 >= target_s:
                break
        return done_bytes, time.perf_counter() - t0, passes


def cpu_baseline(batch, target_s=12.0, max_workers=16):
    """The CPU oracle (fp64 NumPy) on a bounded sample of the same step, on
    every core this process may run on (at most 16 workers, one BLAS thread
    each, fresh interpreters started before the GPU is touched): per level,
    encode each linear input and compute the layer product on the first 512
    rows of each weight shape; whole-host bytes / the slowest worker's time."""
    import multiprocessing as mp

    host = len(os.sched_getaffinity(0))
    workers = max(1, min(host, max_workers))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        res = pool.map(_cpu_worker, [(batch, target_s, i) for i in range(workers)])
    total = sum(r[0] for r in res)
    dt = max(r[1] for r in res)
    passes = sum(r[2] for r in res)
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "host_cores": host,
            "blas_threads": 1, "kind": "oracle",
            "sample": f"{workers} processes x 1 BLAS thread, {passes} pass(es) in total x 12 GEMVs: first 512 rows "
                      f"of each weight shape x levels 2/4/6, batch {batch}, online activation encode; "
                      f"{dt:.1f} s, fp64 NumPy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--pool-layers", type=int, default=9)
    ap.add_argument("--secondary-batch", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-batches", action="store_true", help="skip the batch-16/64 and 70B-shape GEMV lines")
    ap.add_argument("--no-step32", action="store_true", help="skip the 32-layer policy-driven step")
    ap.add_argument("--no-kv", action="store_true", help="skip the KV-cache decode attention line")
    ap.add_argument("--no-formats", action="store_true", help="skip the format-variant comparison lines")
    ap.add_argument("--no-gptq", action="store_true", help="skip the GPTQ calibration line")
    ap.add_argument("--kv-only", action="store_true", help="run only the KV-cache attention (no JSON line)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only the workload of the HBM-counter runs (no JSON line)")
    ap.add_argument("--pmc-batch", action="store_true",
                    help="run only the workload of the 64-token counter runs (no JSON line)")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="run only the prefill GEMM counter workload (no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, so --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    if args.pool_layers % len(LEVELS):
        raise SystemExit("--pool-layers must be a multiple of 3")

    import torch

    import runtime_mixed_precision_amd as A
    from runtime_mixed_precision_amd import synthetic as S

    device = "cuda:0"
    A._native.lib()
    # the CPU baseline first: its worker processes start before this process
    # touches the GPU
    cpu = None
    profiled = any(k.startswith("ROCPROF") for k in os.environ)
    if not args.no_cpu_baseline and not args.pmc_pass and not args.pmc_batch and not args.pmc_prefill and not args.kv_only and not profiled:
        cpu = cpu_baseline(args.batch)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.pmc_pass:
        pmc_pass(A, S, device)
        return
    if args.pmc_batch:
        pmc_batch_pass(A, S, device)
        return
    if args.pmc_prefill:
        pmc_prefill_pass(A, S, device)
        return
    if args.kv_only:
        log(json.dumps(kv_bench(A, S, device, reps=max(args.steps, 5))))
        return
    pool = build_pool(A, S, args.pool_layers, device)
    pool_bytes = sum(w_bytes(wp, 6) for layer in pool for wp in layer.values())
    G = args.pool_layers // len(LEVELS)

    bench = DecodeBench(A, S, pool, args.batch, device)
    graphs = capture([lambda s=s: bench.step(s) for s in range(G)])
    ms_step = time_graphs(graphs, args.steps, args.warmup)
    step_bytes = bench.step_bytes()
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"step: {ms_step:.4f} ms, {step_bytes / 1e6:.1f} MB, {value:.1f} GB/s")
    ugraphs = capture([lambda s=s: bench.step_unfused(s) for s in range(G)])
    ms_unf = time_graphs(ugraphs, args.steps, args.warmup)
    del ugraphs
    log(f"same step without the producer epilogue: {ms_unf:.4f} ms")

    # roofline of the GEMV kernel: GEMV-only graphs, same weights and levels
    ggraphs = capture([lambda s=s: bench.gemv_only(s) for s in range(G)])
    ms_g = time_graphs(ggraphs, max(args.steps, 10), args.warmup)
    n_launch = len(LEVELS) * len(SHAPES)
    g_bytes = bench.gemv_only_bytes()
    achieved = g_bytes / (ms_g * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                "kernel": "gemv_fp4_kernel (one token)",
                "avg_launch_us": round(ms_g * 1e3 / n_launch, 3),
                "bytes_per_launch": int(g_bytes / n_launch)}
    log(f"gemv-only: {ms_g:.4f} ms per {n_launch} launches, {achieved:.1f} GB/s")

    extra = {"step_unfused": {"ms": round(ms_unf, 5), "gbs": round(step_bytes / (ms_unf * 1e-3) / 1e9, 1),
                              "note": "the same chained step with torch elementwise kernels and a separate "
                                      "encode per linear input instead of autofp_epilogue_quantize"}}
    if not args.no_breakdown:
        br = {}
        for name, n, k in SHAPES:
            for level in LEVELS:
                fns = [lambda i=i, name=name, level=level: A.gemv(
                    pool[i][name], bench.xq_l[(name, level)], bits=level, out=bench.y[name],
                    workspace=bench.gws[k]) for i in range(args.pool_layers)]
                g = capture([lambda: [f() for f in fns]])
                ms = time_graphs(g, 10, 2) / args.pool_layers
                gb = gemv_bytes(pool[0][name], args.batch, level) / (ms * 1e-3) / 1e9
                br[f"{name}_l{level}"] = {"us": round(ms * 1e3, 2), "gbs": round(gb, 1)}
        extra["gemv_breakdown_b%d" % args.batch] = br
    if args.secondary_batch and args.secondary_batch != args.batch:
        b2 = DecodeBench(A, S, pool, args.secondary_batch, device)
        g2 = capture([lambda s=s: b2.gemv_only(s) for s in range(G)])
        ms2 = time_graphs(g2, max(args.steps, 10), args.warmup)
        extra[f"gemv_b{args.secondary_batch}"] = {
            "gbs": round(b2.gemv_only_bytes() / (ms2 * 1e-3) / 1e9, 1),
            "avg_launch_us": round(ms2 * 1e3 / n_launch, 3)}
        s2 = capture([lambda s=s: b2.step(s) for s in range(G)])
        ms2s = time_graphs(s2, args.steps, args.warmup)
        extra[f"step_b{args.secondary_batch}"] = {
            "ms": round(ms2s, 4), "gbs": round(b2.step_bytes() / (ms2s * 1e-3) / 1e9, 1)}
        del b2, g2, s2
    if not args.no_batches:
        # the 32-layer step's larger batches: GEMV-only rate over the same 12 launches
        for bb in (16, 64):
            b3 = DecodeBench(A, S, pool, bb, device)
            g3 = capture([lambda s=s: b3.gemv_only(s) for s in range(G)])
            ms3 = time_graphs(g3, 10, args.warmup)
            extra[f"gemv_b{bb}"] = {"gbs": round(b3.gemv_only_bytes() / (ms3 * 1e-3) / 1e9, 1),
                                    "avg_launch_us": round(ms3 * 1e3 / n_launch, 3)}
            del b3, g3
        extra["gemv_70b_b64"] = gemv_70b(A, S, device)
    if not args.no_prefill:
        del graphs, ggraphs
        extra["prefill_gemm"] = prefill_bench(A, S, device, 5)
    if not args.no_formats:
        torch.cuda.empty_cache()
        extra["formats"] = formats_bench(A, S, device)
    if not args.no_gptq:
        torch.cuda.empty_cache()
        extra["gptq"] = gptq_bench(A, S, device)
    if not args.no_step32:
        del pool, bench
        torch.cuda.empty_cache()
        extra["step32"] = step32_bench(A, S, device)
    if not args.no_kv:
        torch.cuda.empty_cache()
        extra["kv_attention"] = kv_bench(A, S, device)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "dtype_note": "E2M1 codes on the fp4 scaled MFMA with E4M3 group scales applied in fp32 (batch-1 GEMV); "
                      "encode in fp32; 16+ tokens and prefill decode the operands to fp16 (exact) for the fp16 MFMA",
        "data": "synthetic",
        "config": {
            "workload": "AutoFP decode step over Llama-3-8B-shaped layers (Wqkv 6144x4096, Wo 4096x4096, "
                        "Wgate|Wup 28672x4096, Wdown 4096x14336): G_E over 128256 logits, then 3 chained layers "
                        "at levels 2/4/6, each: 4 GEMVs, each output post-processed into the next input by one "
                        "producer-epilogue call (copy / residual add + RMSNorm / SwiGLU + AutoFP encode), the last "
                        "one with L_A and the policy update",
            "batch": args.batch,
            "pool_layers": args.pool_layers,
            "pool_bytes": int(pool_bytes),
            "step_bytes": int(step_bytes),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "frac_hbm_peak": round(value / PEAK_HBM_GBS, 4),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
