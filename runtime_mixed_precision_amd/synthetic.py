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
