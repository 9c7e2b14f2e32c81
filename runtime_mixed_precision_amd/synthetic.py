"""Seeded synthetic inputs with the shapes and value distributions of the
AutoFP workloads. Random numbers only; none of the method's arithmetic.

Every tensor is drawn from its own ``torch.Generator`` seeded with
``seed * 1_000_003 + tensor_id`` on the requested device, so the same call
gives the same tensor every time on that device type.
"""

from __future__ import annotations

import torch

# Llama-3-8B-shaped linear layers (out x in)
LLAMA8B = {
    "wqkv": (6144, 4096),
    "wo": (4096, 4096),
    "wgate": (14336, 4096),
    "wup": (14336, 4096),
    "wdown": (4096, 14336),
}
HIDDEN = 4096
FFN = 14336
VOCAB = 128256


def _gen(seed, tensor_id, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tensor_id))
    return g


def activations(rows, k, seed=0, tensor_id=0, outlier_frac=0.01, outlier_scale=20.0,
                dtype=torch.bfloat16, device="cpu"):
    """N(0, 1) activations with a fraction of entries (chosen without
    replacement) multiplied by ``outlier_scale``, rounded to ``dtype``."""
    g = _gen(seed, tensor_id, device)
    x = torch.randn(rows, k, generator=g, device=device, dtype=torch.float32)
    n_out = int(round(outlier_frac * rows * k))
    if n_out:
        idx = torch.randperm(rows * k, generator=g, device=device)[:n_out]
        x.view(-1)[idx] *= outlier_scale
    return x.to(dtype)


def weights(n, k, seed=0, tensor_id=0, std=0.02, heavy_frac=0.01, nu=4.0, device="cpu"):
    """std * N(0, 1) weights [n x k] (fp32) where a fraction of the K-columns
    is drawn from std * Student-t(nu) instead (heavy-tailed input channels).
    Student-t samples are formed as N / sqrt(chi2_nu / nu), chi2 from nu
    squared normals (nu integer)."""
    g = _gen(seed, tensor_id, device)
    w = torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std
    n_heavy = int(round(heavy_frac * k))
    if n_heavy:
        cols = torch.randperm(k, generator=g, device=device)[:n_heavy]
        z = torch.randn(n, n_heavy, generator=g, device=device)
        chi2 = torch.zeros(n, n_heavy, device=device)
        for _ in range(int(nu)):
            chi2 += torch.randn(n, n_heavy, generator=g, device=device) ** 2
        w[:, cols] = std * z / torch.sqrt(chi2 / nu)
    return w


def logits(batch, vocab=VOCAB, seed=0, tensor_id=0, scale=3.0, device="cpu"):
    """Next-token logits ~ scale * N(0, 1), fp32 [batch x vocab]."""
    g = _gen(seed, tensor_id, device)
    return torch.randn(batch, vocab, generator=g, device=device, dtype=torch.float32) * scale


def hidden(batch, dim=HIDDEN, seed=0, tensor_id=0, dtype=torch.float32, device="cpu"):
    """Hidden states ~ N(0, 1) [batch x dim]."""
    g = _gen(seed, tensor_id, device)
    return torch.randn(batch, dim, generator=g, device=device, dtype=torch.float32).to(dtype)


def calibration(tokens, k, seed=0, tensor_id=0, corr=0.8, device="cpu"):
    """Calibration activations [tokens x k] fp32 whose neighbouring channels
    are correlated: x[:, 0] = z[:, 0], x[:, i] = corr * x[:, i-1] +
    sqrt(1 - corr^2) * z[:, i] with z ~ N(0, 1) (unit variance per channel),
    a stand-in for the activations a calibration set would give."""
    g = _gen(seed, tensor_id, device)
    z = torch.randn(tokens, k, generator=g, device=device, dtype=torch.float32)
    x = torch.empty_like(z)
    x[:, 0] = z[:, 0]
    c = (1.0 - corr * corr) ** 0.5
    for i in range(1, k):
        x[:, i] = corr * x[:, i - 1] + c * z[:, i]
    return x


def kv_tokens(n, h_kv, head_dim=128, seed=0, tensor_id=0, dtype=torch.bfloat16, device="cpu"):
    """K or V vectors ~ N(0, 1) [n x h_kv x head_dim], rounded to ``dtype``."""
    g = _gen(seed, tensor_id, device)
    return torch.randn(n, h_kv, head_dim, generator=g, device=device, dtype=torch.float32).to(dtype)


def kv_page_plan(lengths, refine_frac=0.0, seed=0, max_run=96, page_tokens=64):
    """A page layout for sequences of the given token counts (host bookkeeping).

    Each sequence's tokens come in runs of 1 .. max_run tokens; a run is
    refined with probability ``refine_frac`` (all runs refined for 1.0, none
    for 0.0). A sequence keeps one open page per type (base: page_tokens
    tokens, refinement: page_tokens / 2) and opens a new one when it fills.
    Page ids are a random permutation, so a sequence's pages are scattered.

    Returns a dict of numpy arrays: page_kind [n_pages] uint8, page_tokens
    [n_pages] int32, page_table [batch, max_pages] int32 (-1 padded),
    seq_pages [batch] int32, and per sequence: slots (page * page_tokens +
    position per token, in token order) and refine (bool per token).
    """
    import numpy as np

    rng = np.random.default_rng([int(seed), 7])
    kinds, fills, owners = [], [], []
    seq_slots, seq_refine, seq_pages_l = [], [], []
    for b, L in enumerate(lengths):
        ref = np.zeros(L, dtype=bool)
        if refine_frac >= 1.0:
            ref[:] = True
        elif refine_frac > 0.0:
            t = 0
            while t < L:
                run = int(rng.integers(1, max_run + 1))
                ref[t:t + run] = rng.random() < refine_frac
                t += run
        open_page = {0: -1, 1: -1}
        slots = np.empty(L, dtype=np.int64)
        pages = []
        for t in range(L):
            kd = int(ref[t])
            cap = page_tokens // 2 if kd else page_tokens
            p = open_page[kd]
            if p < 0 or fills[p] == cap:
                p = len(kinds)
                kinds.append(kd)
                fills.append(0)
                owners.append(b)
                open_page[kd] = p
                pages.append(p)
            slots[t] = p * page_tokens + fills[p]
            fills[p] += 1
        seq_slots.append(slots)
        seq_refine.append(ref)
        seq_pages_l.append(pages)
    n_pages = max(len(kinds), 1)
    perm = rng.permutation(n_pages)           # logical page -> physical id
    page_kind = np.zeros(n_pages, np.uint8)
    page_fill = np.zeros(n_pages, np.int32)
    for p in range(len(kinds)):
        page_kind[perm[p]] = kinds[p]
        page_fill[perm[p]] = fills[p]
    max_pages = max(1, max(len(p) for p in seq_pages_l))
    table = np.full((len(lengths), max_pages), -1, np.int32)
    for b, pages in enumerate(seq_pages_l):
        table[b, :len(pages)] = perm[np.asarray(pages, dtype=np.int64)] if pages else []
    out_slots = []
    for slots in seq_slots:
        p, pos = slots // page_tokens, slots % page_tokens
        out_slots.append((perm[p] * page_tokens + pos).astype(np.int32) if len(slots) else slots.astype(np.int32))
    return dict(page_kind=page_kind, page_tokens=page_fill, page_table=table,
                seq_pages=np.array([len(p) for p in seq_pages_l], np.int32),
                slots=out_slots, refine=seq_refine, n_pages=n_pages, max_pages=max_pages)
