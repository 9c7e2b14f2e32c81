"""AutoFP block-scaled low-bit linear layer on MI355X (gfx950).

Thin PyTorch-facing binding over the C ABI of ``include/autofp.h``
(``libautofp.so``): it allocates device buffers with torch, marshals pointers
and sizes, and calls the library on torch's current stream. Every step of the
computation runs in the library's HIP kernels; if the library is missing the
calls raise ``NativeLibraryError``.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import torch

from . import _native as N
from ._native import AutofpError, NativeLibraryError, Params  # noqa: F401

__all__ = [
    "AutoFPTensor", "default_params", "packed_bytes", "weight_refined_count", "workspace_bytes",
    "select_weight_mask", "quantize", "quantize_weight", "quantize_activation",
    "alloc_activation", "quantize_into", "quantize_noalloc", "epilogue_quantize", "gptq_quantize",
    "gemv", "gemv_rows", "gemm", "policy_signals", "policy_state", "policy_update", "AutofpError",
    "NativeLibraryError", "KVCache", "kv_write", "kv_attention", "layer_epilogue", "policy_layer",
    "save_packed", "load_packed",
]

_DT = {torch.float32: N.F32, torch.bfloat16: N.BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def default_params(**overrides) -> Params:
    p = Params()
    N.check(N.lib().autofp_default_params(C.byref(p)), "autofp_default_params")
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def _fmt(format) -> int:
    """autofp_format code of a format name ("autofp6", "autofp6e", "autofp8",
    "fp6g") or code."""
    if isinstance(format, str):
        if format not in N.FORMATS:
            raise ValueError(f"unknown format {format!r}; one of {sorted(N.FORMATS)}")
        return N.FORMATS[format]
    return int(format)


def packed_bytes(rows, k, kind, refine=False, n_refined=0, format="autofp6"):
    out = (C.c_size_t * 5)()
    N.check(N.lib().autofp_packed_bytes(rows, k, kind, _fmt(format), int(bool(refine)), n_refined, out),
            "autofp_packed_bytes")
    return list(out)


def weight_refined_count(k, params=None) -> int:
    p = params or default_params()
    n = C.c_int32()
    N.check(N.lib().autofp_weight_refined_count(k, C.byref(p), C.byref(n)),
            "autofp_weight_refined_count")
    return int(n.value)


def workspace_bytes(op, rows, k) -> int:
    b = C.c_size_t()
    N.check(N.lib().autofp_workspace_bytes(op, rows, k, C.byref(b)), "autofp_workspace_bytes")
    return int(b.value)


def _workspace(op, rows, k, device):
    return torch.empty(max(workspace_bytes(op, rows, k), 16), dtype=torch.uint8, device=device)


@dataclass
class AutoFPTensor:
    """Device buffers of one packed AutoFP tensor (layout of include/autofp.h)."""
    rows: int
    k: int
    kind: int
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    mask: Optional[torch.Tensor] = None
    offsets: Optional[torch.Tensor] = None
    n_refined: int = 0
    format: int = 0     # autofp_format

    def struct(self) -> N.Packed:
        return N.Packed(self.rows, self.k, self.kind, self.n_refined, _ptr(self.codes),
                        _ptr(self.scales), _ptr(self.tensor_scale), _ptr(self.mask),
                        _ptr(self.offsets), self.format, 0)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.codes, self.scales, self.tensor_scale, self.mask, self.offsets)
                   if t is not None)

    def to_host(self) -> dict:
        """Host copy in the packed-format dictionary layout used by the tests."""
        d = dict(codes=self.codes.cpu().numpy(), scales=self.scales.cpu().numpy(),
                 T=self.tensor_scale.cpu().numpy()[0], rows=self.rows, k=self.k)
        if self.mask is not None:
            d["mask"] = self.mask.cpu().numpy()
        if self.offsets is not None:
            d["offsets"] = self.offsets.cpu().numpy()
        if self.kind == N.WEIGHT:
            d["n_refined"] = self.n_refined
        d["format"] = self.format
        return d


def _alloc_packed(rows, k, kind, refine, n_refined, device, format=0):
    fmt = _fmt(format)
    nb = packed_bytes(rows, k, kind, refine, n_refined, fmt)

    def buf(n, shape):
        return torch.zeros(shape, dtype=torch.uint8, device=device) if n else None

    mb = (k + 31) // 32
    ow = 2 if fmt == N.FMT_AUTOFP8 else 1       # offset bytes per subgroup
    codes = torch.empty(rows, nb[0] // rows, dtype=torch.uint8, device=device)
    scales = torch.empty(rows, k // 16, dtype=torch.uint8, device=device)
    ts = torch.empty(1, dtype=torch.float32, device=device)
    if kind == N.WEIGHT:
        mask = buf(nb[3], (mb,))
        offs = None
        if refine:
            # rows x n_refined offset words plus the padding the GEMV may read past the end
            flat = torch.zeros(max(nb[4], rows * n_refined * ow + 16), dtype=torch.uint8, device=device)
            offs = flat[: rows * n_refined * ow].view(rows, n_refined * ow)
    else:
        mask = buf(nb[3], (rows, mb))
        offs = buf(nb[4], (rows, (k // 4) * ow))
    return AutoFPTensor(rows, k, kind, codes, scales, ts, mask, offs, n_refined if kind == N.WEIGHT else 0, fmt)


_SAVE_VERSION = "1"
_SAVE_FIELDS = ("codes", "scales", "tensor_scale", "mask", "offsets")


def save_packed(path, tensors: dict) -> None:
    """Write packed tensors (name -> AutoFPTensor) to a safetensors file.

    Each buffer is stored as-is (byte codes, E4M3 scale bytes, the fp32 tensor
    scale, mask and offset bytes) under ``<name>.<field>``; rows, k, kind,
    n_refined and the format go into the file's string metadata. Nothing is
    re-encoded, so a loaded tensor gives bit-identical GEMV/GEMM outputs.
    """
    from safetensors.torch import save_file
    blobs, meta = {}, {"autofp_packed_version": _SAVE_VERSION}
    for name, t in tensors.items():
        if "." in name:
            raise ValueError(f"tensor name {name!r} may not contain '.'")
        meta[name] = f"{t.rows},{t.k},{t.kind},{t.n_refined},{t.format}"
        for f in _SAVE_FIELDS:
            b = getattr(t, f)
            if b is not None:
                blobs[f"{name}.{f}"] = b.detach().contiguous().cpu()
    save_file(blobs, str(path), metadata=meta)


def load_packed(path, device="cuda:0") -> dict:
    """Read a file written by ``save_packed``: name -> AutoFPTensor on ``device``.

    The buffers are allocated as the quantizers allocate them (including the
    padding after a weight's offsets that the GEMV may read) and filled from
    the file; a buffer whose size or dtype differs from what the metadata
    implies, or a file safetensors cannot parse, raises ``ValueError``. The
    file is parsed by safetensors, which executes nothing from it.
    """
    from safetensors import SafetensorError, safe_open
    try:
        return _load_packed(safe_open(str(path), framework="pt", device="cpu"), path, device)
    except SafetensorError as e:
        raise ValueError(f"{path}: {e}") from None


def _load_packed(handle, path, device):
    out = {}
    with handle as f:
        meta = f.metadata() or {}
        if meta.get("autofp_packed_version") != _SAVE_VERSION:
            raise ValueError(f"{path}: not an AutoFP packed file (version {meta.get('autofp_packed_version')!r})")
        keys = set(f.keys())
        for name, desc in meta.items():
            if name == "autofp_packed_version":
                continue
            try:
                rows, k, kind, n_ref, fmt = (int(v) for v in desc.split(","))
            except ValueError:
                raise ValueError(f"{path}: bad metadata for {name!r}: {desc!r}") from None
            refine = f"{name}.offsets" in keys
            t = _alloc_packed(rows, k, kind, refine, n_ref, device, fmt)
            for fld in _SAVE_FIELDS:
                dst, key = getattr(t, fld), f"{name}.{fld}"
                if (dst is None) != (key not in keys):
                    raise ValueError(f"{path}: {key} is {'missing' if dst is not None else 'unexpected'}")
                if dst is None:
                    continue
                src = f.get_tensor(key)
                if src.dtype != dst.dtype or tuple(src.shape) != tuple(dst.shape):
                    raise ValueError(f"{path}: {key} has {src.dtype} {tuple(src.shape)}, "
                                     f"expected {dst.dtype} {tuple(dst.shape)}")
                dst.copy_(src)
            out[name] = t
    return out


def select_weight_mask(w: torch.Tensor, params=None, stream=None, format="autofp6"):
    """Weight mask M_W (device uint8 [ceil(k/32)]) and its refined-subgroup
    count, with the gains of ``format``'s offsets."""
    _dev_check(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("weight must be a 2-D float32 tensor")
    p = params or default_params()
    rows, k = w.shape
    mask = torch.zeros((k + 31) // 32, dtype=torch.uint8, device=w.device)
    ws = _workspace(N.OP_SELECT_MASK, rows, k, w.device)
    N.check(N.lib().autofp_select_weight_mask(_ptr(w), rows, k, _fmt(format), C.byref(p), _ptr(mask), _ptr(ws),
                                              ws.numel(), _stream(stream)), "autofp_select_weight_mask")
    return mask, weight_refined_count(k, p)


def quantize(x: torch.Tensor, kind: int, refine=False, exclude_mask=None, weight_mask=None,
             n_refined=0, params=None, stream=None, format="autofp6") -> AutoFPTensor:
    """Encode a [rows x k] fp32/bf16 tensor to AutoFP (autofp_quantize) in
    ``format`` ("autofp6", "autofp6e", "autofp8" or "fp6g")."""
    _dev_check(x, exclude_mask, weight_mask)
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be a 2-D float32 or bfloat16 tensor")
    rows, k = x.shape
    p = params or default_params()
    if kind == N.WEIGHT:
        out = _alloc_packed(rows, k, kind, weight_mask is not None, n_refined, x.device, format)
        if weight_mask is not None:
            out.mask = weight_mask
    else:
        out = _alloc_packed(rows, k, kind, refine, 0, x.device, format)
    ws = _workspace(N.OP_QUANTIZE, rows, k, x.device)
    st = out.struct()
    N.check(N.lib().autofp_quantize(_ptr(x), _DT[x.dtype], int(bool(refine)), _ptr(exclude_mask),
                                    C.byref(p), C.byref(st), _ptr(ws), ws.numel(), _stream(stream)),
            "autofp_quantize")
    return out


def alloc_activation(rows, k, refine=True, device="cuda:0", format="autofp6") -> AutoFPTensor:
    """Device buffers for a [rows x k] activation (with refinement storage)."""
    return _alloc_packed(rows, k, N.ACTIVATION, refine, 0, device, format)


def quantize_into(x: torch.Tensor, out: AutoFPTensor, refine=False, exclude_mask=None,
                  workspace=None, params=None, stream=None) -> AutoFPTensor:
    """autofp_quantize into preallocated buffers (no allocation; graph-safe
    when ``workspace`` is given)."""
    if x.dim() != 2 or x.dtype not in _DT or tuple(x.shape) != (out.rows, out.k):
        raise ValueError("x must be 2-D float32/bfloat16 with the output's shape")
    p = params or default_params()
    if workspace is None:
        workspace = _workspace(N.OP_QUANTIZE, out.rows, out.k, x.device)
    st = out.struct()
    N.check(N.lib().autofp_quantize(_ptr(x), _DT[x.dtype], int(bool(refine)), _ptr(exclude_mask),
                                    C.byref(p), C.byref(st), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "autofp_quantize")
    return out


def epilogue_quantize(op, z: torch.Tensor, out: AutoFPTensor, residual=None, v_out=None, refine=False,
                      exclude_mask=None, workspace=None, params=None, stream=None) -> AutoFPTensor:
    """autofp_epilogue_quantize: v = op(z) (``"copy"``: the first out.k columns
    of z; ``"residual"``: residual + z; ``"swiglu"``: silu(z[:, :k]) *
    z[:, k:2k]; ``"residual_rmsnorm"``: RMSNorm(residual + z), with v_out
    receiving the residual sum itself) in fp32, written to ``v_out`` when
    given, and encoded into ``out`` as autofp_quantize encodes v. A given
    ``workspace`` holds workspace_bytes(OP_EPILOGUE, out.rows, out.k) bytes."""
    ops = {"copy": N.EPI_COPY, "residual": N.EPI_RESIDUAL, "swiglu": N.EPI_SWIGLU,
           "residual_rmsnorm": N.EPI_RESIDUAL_RMSNORM}
    _dev_check(residual, v_out, exclude_mask)
    if z.dtype != torch.float32 or z.dim() != 2 or z.stride(1) != 1 or z.shape[0] != out.rows:
        raise ValueError("z must be a 2-D float32 tensor with unit column stride and out.rows rows")
    p = params or default_params()
    if workspace is None:
        workspace = _workspace(N.OP_EPILOGUE, out.rows, out.k, z.device)
    st = out.struct()
    N.check(N.lib().autofp_epilogue_quantize(ops[op], _ptr(z), z.stride(0), _ptr(residual), _ptr(v_out),
                                             int(bool(refine)), _ptr(exclude_mask), C.byref(p), C.byref(st),
                                             _ptr(workspace), workspace.numel(), _stream(stream)),
            "autofp_epilogue_quantize")
    return out


def layer_epilogue(z: torch.Tensor, out: AutoFPTensor, residual, v_out, h_prev, phase, layer, state,
                   g_e=None, new_sequence=False, l_a=None, bits_rows=None, bits_layer=None, refine=False,
                   exclude_mask=None, workspace=None, params=None, stream=None):
    """autofp_layer_epilogue: the layer's last producer epilogue (residual add
    into ``v_out``, its RMSNorm encoded into ``out``) and the layer's policy
    step (L_A from ``h_prev`` and the new hidden state, then Table 1) in one
    call. Returns (l_a [rows] fp32, bits_rows [rows] int32, bits_layer [1]
    int32). A given ``workspace`` holds workspace_bytes(OP_EPILOGUE, rows, k)."""
    _dev_check(residual, v_out, h_prev, g_e, state, exclude_mask)
    if z.dtype != torch.float32 or z.dim() != 2 or z.stride(1) != 1 or z.shape[0] != out.rows:
        raise ValueError("z must be a 2-D float32 tensor with unit column stride and out.rows rows")
    for t in (residual, v_out, h_prev):
        if t is None or t.dtype != torch.float32 or tuple(t.shape) != (out.rows, out.k) or not t.is_contiguous():
            raise ValueError("residual, v_out and h_prev must be contiguous float32 [rows, k] tensors")
    dev = z.device
    if l_a is None:
        l_a = torch.empty(out.rows, dtype=torch.float32, device=dev)
    if bits_rows is None:
        bits_rows = torch.empty(out.rows, dtype=torch.int32, device=dev)
    if bits_layer is None:
        bits_layer = torch.empty(1, dtype=torch.int32, device=dev)
    p = params or default_params()
    if workspace is None:
        workspace = _workspace(N.OP_EPILOGUE, out.rows, out.k, dev)
    st = out.struct()
    N.check(N.lib().autofp_layer_epilogue(_ptr(z), z.stride(0), _ptr(residual), _ptr(v_out), _ptr(h_prev),
                                          int(bool(refine)), _ptr(exclude_mask), int(phase), int(layer),
                                          int(bool(new_sequence)), _ptr(g_e), C.byref(p), _ptr(state), _ptr(l_a),
                                          _ptr(bits_rows), _ptr(bits_layer), C.byref(st), _ptr(workspace),
                                          workspace.numel(), _stream(stream)),
            "autofp_layer_epilogue")
    return l_a, bits_rows, bits_layer


def quantize_noalloc(x: torch.Tensor, out: AutoFPTensor, refine=False, exclude_mask=None, params=None,
                     stream=None) -> AutoFPTensor:
    """autofp_quantize_noalloc into preallocated buffers: no workspace, the
    library's static per-GPU scratch instead (k <= 491488; calls that overlap
    on one GPU race)."""
    _dev_check(x, exclude_mask)
    if x.dim() != 2 or x.dtype not in _DT or tuple(x.shape) != (out.rows, out.k):
        raise ValueError("x must be 2-D float32/bfloat16 with the output's shape")
    p = params or default_params()
    st = out.struct()
    N.check(N.lib().autofp_quantize_noalloc(_ptr(x), _DT[x.dtype], int(bool(refine)), _ptr(exclude_mask),
                                            C.byref(p), C.byref(st), _stream(stream)),
            "autofp_quantize_noalloc")
    return out


def quantize_weight(w: torch.Tensor, refine=True, params=None, stream=None, format="autofp6") -> AutoFPTensor:
    """Offline weight packing: M_W selection (when ``refine``) and encode."""
    if refine and _fmt(format) != N.FMT_FP6G:
        mask, nref = select_weight_mask(w, params, stream, format)
        return quantize(w, N.WEIGHT, refine=True, weight_mask=mask, n_refined=nref, params=params,
                        stream=stream, format=format)
    return quantize(w, N.WEIGHT, params=params, stream=stream, format=format)


def gptq_quantize(w: torch.Tensor, u: torch.Tensor, h_diag: torch.Tensor, params=None, workspace=None,
                  stream=None) -> AutoFPTensor:
    """Refinement-aware GPTQ (autofp_gptq_quantize): w [rows x k] fp32, u
    [k x k] fp64 upper Cholesky factor of the inverse Hessian, h_diag [k]
    fp64 Hessian diagonal; returns the packed AutoFP6 weight with its mask."""
    _dev_check(w, u, h_diag)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    rows, k = w.shape
    if u.dtype != torch.float64 or tuple(u.shape) != (k, k) or h_diag.dtype != torch.float64 or h_diag.numel() != k:
        raise ValueError("u must be float64 [k, k] and h_diag float64 [k]")
    p = params or default_params()
    nref = weight_refined_count(k, p)
    out = _alloc_packed(rows, k, N.WEIGHT, True, nref, w.device)
    if workspace is None:
        workspace = _workspace(N.OP_GPTQ, rows, k, w.device)
    st = out.struct()
    N.check(N.lib().autofp_gptq_quantize(_ptr(w), rows, k, _ptr(u), _ptr(h_diag), C.byref(p), C.byref(st),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
            "autofp_gptq_quantize")
    return out


def quantize_activation(x: torch.Tensor, refine=False, exclude_mask=None, params=None,
                        stream=None, format="autofp6") -> AutoFPTensor:
    return quantize(x, N.ACTIVATION, refine=refine, exclude_mask=exclude_mask, params=params,
                    stream=stream, format=format)


def _linear(fn, name, w, x, bits, bits_dev, out_dtype, params, workspace, out, stream):
    _dev_check(bits_dev)
    p = params or default_params()
    op = N.OP_GEMV if name == "autofp_gemv" else N.OP_GEMM
    if out is None:
        out = torch.empty(x.rows, w.rows, dtype=out_dtype, device=w.codes.device)
    if workspace is None:
        workspace = _workspace(op, x.rows, x.k, w.codes.device)
    ws_, xs_ = w.struct(), x.struct()
    N.check(fn(C.byref(ws_), C.byref(xs_), int(bits), _ptr(bits_dev), _ptr(out), _DT[out.dtype],
               C.byref(p), _ptr(workspace), workspace.numel(), _stream(stream)), name)
    return out


def gemv(w: AutoFPTensor, x: AutoFPTensor, bits=4, bits_dev=None, out_dtype=torch.float32,
         params=None, workspace=None, out=None, stream=None) -> torch.Tensor:
    """y = Xhat . What^T at level ``bits`` (decode path, autofp_gemv)."""
    return _linear(N.lib().autofp_gemv, "autofp_gemv", w, x, bits, bits_dev, out_dtype, params,
                   workspace, out, stream)


def gemv_rows(w: AutoFPTensor, x: AutoFPTensor, bits_rows: torch.Tensor, out_dtype=torch.float32,
              params=None, workspace=None, out=None, stream=None) -> torch.Tensor:
    """y = Xhat . What^T with row b at level ``bits_rows[b]`` (int32 device
    tensor of 2/4/6 per token; autofp_gemv_rows)."""
    _dev_check(bits_rows)
    if bits_rows.dtype != torch.int32 or bits_rows.numel() != x.rows:
        raise ValueError("bits_rows must be int32 with one level per activation row")
    p = params or default_params()
    if out is None:
        out = torch.empty(x.rows, w.rows, dtype=out_dtype, device=w.codes.device)
    if workspace is None:
        workspace = _workspace(N.OP_GEMV, x.rows, x.k, w.codes.device)
    ws_, xs_ = w.struct(), x.struct()
    N.check(N.lib().autofp_gemv_rows(C.byref(ws_), C.byref(xs_), _ptr(bits_rows), _ptr(out), _DT[out.dtype],
                                     C.byref(p), _ptr(workspace), workspace.numel(), _stream(stream)),
            "autofp_gemv_rows")
    return out


def gemm(w: AutoFPTensor, x: AutoFPTensor, bits=4, bits_dev=None, out_dtype=torch.float32,
         params=None, workspace=None, out=None, stream=None) -> torch.Tensor:
    """y = Xhat . What^T at level ``bits`` (prefill path, autofp_gemm)."""
    return _linear(N.lib().autofp_gemm, "autofp_gemm", w, x, bits, bits_dev, out_dtype, params,
                   workspace, out, stream)


def policy_signals(logits=None, h_prev=None, h_cur=None, params=None, stream=None,
                   out_entropy=None, out_update=None, workspace=None):
    """(G_E per row or None, L_A per row or None) via autofp_policy_signals.

    ``workspace`` (uint8 device tensor of workspace_bytes(OP_SIGNALS, batch,
    vocab) bytes) is allocated per call when not given; pass one to keep the
    call free of allocations (e.g. under graph capture)."""
    _dev_check(logits, h_prev, h_cur)
    p = params or default_params()
    ent = upd = None
    batch = vocab = hidden = 0
    hdt = N.F32
    if logits is not None:
        if logits.dtype != torch.float32 or logits.dim() != 2:
            raise ValueError("logits must be 2-D float32")
        batch, vocab = logits.shape
        ent = out_entropy if out_entropy is not None else \
            torch.empty(batch, dtype=torch.float32, device=logits.device)
        if workspace is None:
            workspace = _workspace(N.OP_SIGNALS, batch, vocab, logits.device)
    if h_prev is not None:
        if h_prev.shape != h_cur.shape or h_prev.dtype != h_cur.dtype or h_prev.dim() != 2:
            raise ValueError("h_prev and h_cur must be matching 2-D tensors")
        if logits is not None and h_prev.shape[0] != batch:
            raise ValueError("logits and hidden states need the same batch")
        batch, hidden = h_prev.shape
        hdt = _DT[h_prev.dtype]
        upd = out_update if out_update is not None else \
            torch.empty(batch, dtype=torch.float32, device=h_prev.device)
    wsb = workspace.numel() if workspace is not None else 0
    N.check(N.lib().autofp_policy_signals(_ptr(logits), batch, vocab, _ptr(h_prev), _ptr(h_cur), hdt,
                                          hidden, C.byref(p), _ptr(ent), _ptr(upd), _ptr(workspace),
                                          wsb, _stream(stream)),
            "autofp_policy_signals")
    return ent, upd


def policy_state(batch, device="cuda:0") -> torch.Tensor:
    """Zero-filled device state for ``batch`` sequences (autofp_policy_state)."""
    return torch.zeros(batch, N.POLICY_STATE_BYTES, dtype=torch.uint8, device=device)


def policy_update(phase, layer, l_a, state, g_e=None, new_sequence=False, bits_rows=None,
                  bits_layer=None, params=None, stream=None):
    """One device-side policy step after ``layer`` (autofp_policy_update).
    phase 0 = prefill, 1 = decode. Returns (bits_rows [batch] int32,
    bits_layer [1] int32), the levels of the next layer."""
    _dev_check(l_a, g_e, state)
    batch = l_a.shape[0]
    if bits_rows is None:
        bits_rows = torch.empty(batch, dtype=torch.int32, device=l_a.device)
    if bits_layer is None:
        bits_layer = torch.empty(1, dtype=torch.int32, device=l_a.device)
    p = params or default_params()
    N.check(N.lib().autofp_policy_update(int(phase), int(layer), int(bool(new_sequence)), _ptr(l_a),
                                         _ptr(g_e), batch, C.byref(p), _ptr(state), _ptr(bits_rows),
                                         _ptr(bits_layer), _stream(stream)), "autofp_policy_update")
    return bits_rows, bits_layer


def policy_layer(phase, layer, h_prev, h_cur, state, g_e=None, new_sequence=False, l_a=None, bits_rows=None,
                 bits_layer=None, params=None, stream=None):
    """L_A of the layer and the policy step in one call (autofp_policy_layer).
    h_prev, h_cur [batch, hidden] fp32 or bf16. Returns (l_a [batch] fp32,
    bits_rows [batch] int32, bits_layer [1] int32)."""
    _dev_check(h_prev, h_cur, g_e, state)
    if h_prev.shape != h_cur.shape or h_prev.dtype != h_cur.dtype or h_prev.dim() != 2:
        raise ValueError("h_prev and h_cur must be matching [batch, hidden] tensors")
    batch, hidden = h_prev.shape
    dev = h_prev.device
    if l_a is None:
        l_a = torch.empty(batch, dtype=torch.float32, device=dev)
    if bits_rows is None:
        bits_rows = torch.empty(batch, dtype=torch.int32, device=dev)
    if bits_layer is None:
        bits_layer = torch.empty(1, dtype=torch.int32, device=dev)
    p = params or default_params()
    N.check(N.lib().autofp_policy_layer(int(phase), int(layer), int(bool(new_sequence)), _ptr(h_prev),
                                        _ptr(h_cur), _DT[h_prev.dtype], hidden, _ptr(g_e), batch, C.byref(p),
                                        _ptr(state), _ptr(l_a), _ptr(bits_rows), _ptr(bits_layer),
                                        _stream(stream)), "autofp_policy_layer")
    return l_a, bits_rows, bits_layer


class KVCache:
    """Device buffers of an AutoFP KV cache (autofp_kv_cache): K and V page
    pools [n_pages][h_kv][4608] bytes, the page types (0 base: 64 tokens,
    1 refinement: 32 refined tokens), the tokens each page holds, the two
    tensor scales and a page table of ``batch`` sequences."""

    def __init__(self, n_pages, h_kv, batch, max_pages, device="cuda:0"):
        dev = torch.device(device)
        self.h_kv, self.n_pages, self.batch, self.max_pages = h_kv, n_pages, batch, max_pages
        self.k_pages = torch.zeros(n_pages, h_kv, N.KV_PAGE_BYTES, dtype=torch.uint8, device=dev)
        self.v_pages = torch.zeros_like(self.k_pages)
        self.page_kind = torch.zeros(n_pages, dtype=torch.uint8, device=dev)
        self.scales = torch.zeros(2, dtype=torch.float32, device=dev)       # T_K, T_V
        self.page_table = torch.full((batch, max_pages), -1, dtype=torch.int32, device=dev)
        self.seq_pages = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.page_tokens = torch.zeros(n_pages, dtype=torch.int32, device=dev)

    def struct(self) -> N.KvCache:
        c = N.KvCache()
        c.h_kv, c.head_dim, c.n_pages, c.max_pages = self.h_kv, N.KV_HEAD_DIM, self.n_pages, self.max_pages
        c.k_pages, c.v_pages = self.k_pages.data_ptr(), self.v_pages.data_ptr()
        c.page_kind = self.page_kind.data_ptr()
        c.k_scale = self.scales.data_ptr()
        c.v_scale = self.scales.data_ptr() + 4
        c.page_table = self.page_table.data_ptr()
        c.seq_pages = self.seq_pages.data_ptr()
        c.page_tokens = self.page_tokens.data_ptr()
        return c


def kv_write(cache: KVCache, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, set_scale=False,
             workspace=None, stream=None):
    """Encode tokens k, v [n, h_kv, 128] (fp32 or bf16) into the pages named by
    ``slots`` [n] int32 (page * 64 + position), autofp_kv_write."""
    _dev_check(k, v, slots)
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3:
        raise ValueError("k and v must be matching [n, h_kv, head_dim] tensors")
    if slots.dtype != torch.int32 or slots.numel() != k.shape[0]:
        raise ValueError("slots must be int32 with one entry per token")
    n = k.shape[0]
    if workspace is None and set_scale:
        workspace = _workspace(N.OP_KV_WRITE, n * cache.h_kv, N.KV_HEAD_DIM, k.device)
    c = cache.struct()
    N.check(N.lib().autofp_kv_write(_ptr(k), _ptr(v), _DT[k.dtype], n, _ptr(slots), int(bool(set_scale)),
                                    C.byref(c), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                    _stream(stream)), "autofp_kv_write")


def kv_attention(q: torch.Tensor, cache: KVCache, bits=4, bits_dev=None, sm_scale=None, out=None,
                 workspace=None, stream=None) -> torch.Tensor:
    """Decode attention of q [batch, h_q, 128] (fp32 or bf16) over the cache,
    autofp_kv_attention; returns [batch, h_q, 128] fp32."""
    _dev_check(q, bits_dev)
    if q.dim() != 3:
        raise ValueError("q must be [batch, h_q, head_dim]")
    batch, h_q, _ = q.shape
    if sm_scale is None:
        sm_scale = N.KV_HEAD_DIM ** -0.5
    if out is None:
        out = torch.empty(batch, h_q, N.KV_HEAD_DIM, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(N.OP_KV_ATTENTION, batch * h_q, cache.max_pages, q.device)
    c = cache.struct()
    N.check(N.lib().autofp_kv_attention(_ptr(q), _DT[q.dtype], batch, h_q, C.byref(c), int(bits),
                                        _ptr(bits_dev), float(sm_scale), _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(stream)), "autofp_kv_attention")
    return out
