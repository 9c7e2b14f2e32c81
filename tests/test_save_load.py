"""Save / load of packed AutoFP tensors (host side): every buffer comes back
byte for byte with its metadata, and malformed files are rejected. Only the
allocator's size query calls the library; no GPU is used."""

import json
import struct

import pytest
import torch

import runtime_mixed_precision_amd as A
from runtime_mixed_precision_amd import _native as N


def _random_packed(rows, k, kind, refine, n_refined, fmt, seed):
    t = A._alloc_packed(rows, k, kind, refine, n_refined, "cpu", fmt)
    g = torch.Generator().manual_seed(seed)
    for f in A._SAVE_FIELDS:
        b = getattr(t, f)
        if b is None:
            continue
        if b.dtype == torch.uint8:
            b.copy_(torch.randint(0, 256, b.shape, dtype=torch.uint8, generator=g))
        else:
            b.copy_(torch.rand(b.shape, generator=g))
    return t


CASES = [
    ("w_plain", 96, 512, N.WEIGHT, False, 0, N.FMT_AUTOFP6),
    ("w_ref", 64, 1024, N.WEIGHT, True, 12, N.FMT_AUTOFP6),
    ("w_ref8", 32, 256, N.WEIGHT, True, 4, N.FMT_AUTOFP8),
    ("x_plain", 5, 512, N.ACTIVATION, False, 0, N.FMT_AUTOFP6),
    ("x_ref", 3, 768, N.ACTIVATION, True, 0, N.FMT_AUTOFP6E),
    ("x_fp6g", 2, 256, N.ACTIVATION, False, 0, N.FMT_FP6G),
]


def test_round_trip_is_byte_exact(tmp_path):
    src = {c[0]: _random_packed(*c[1:], seed=i) for i, c in enumerate(CASES)}
    path = tmp_path / "packed.safetensors"
    A.save_packed(path, src)
    got = A.load_packed(path, device="cpu")
    assert set(got) == set(src)
    for name, t in src.items():
        u = got[name]
        assert (u.rows, u.k, u.kind, u.n_refined, u.format) == (t.rows, t.k, t.kind, t.n_refined, t.format)
        for f in A._SAVE_FIELDS:
            a, b = getattr(t, f), getattr(u, f)
            assert (a is None) == (b is None), (name, f)
            if a is not None:
                assert a.dtype == b.dtype and a.shape == b.shape and torch.equal(a, b), (name, f)
    # a refined weight keeps the readable padding after its offsets
    w = got["w_ref"]
    assert w.offsets.untyped_storage().nbytes() > w.offsets.numel()


def _rewrite_header(path, edit):
    raw = path.read_bytes()
    n = struct.unpack("<Q", raw[:8])[0]
    head = json.loads(raw[8:8 + n])
    edit(head)
    nh = json.dumps(head).encode()
    nh += b" " * (-len(nh) % 8)
    path.write_bytes(struct.pack("<Q", len(nh)) + nh + raw[8 + n:])


@pytest.mark.parametrize("what", ["version", "metadata", "missing", "shape"])
def test_malformed_files_are_rejected(tmp_path, what):
    t = _random_packed(*CASES[1][1:], seed=7)
    path = tmp_path / "bad.safetensors"
    A.save_packed(path, {"w": t})

    def edit(h):
        if what == "version":
            h["__metadata__"]["autofp_packed_version"] = "0"
        elif what == "metadata":
            h["__metadata__"]["w"] = "64,1024"
        elif what == "missing":
            del h["w.offsets"]   # its bytes stay in the data section
        else:
            # claim 16 more weight rows than the buffers hold
            h["__metadata__"]["w"] = "80,1024,0,12,0"
    _rewrite_header(path, edit)
    with pytest.raises(ValueError):
        A.load_packed(path, device="cpu")


def test_field_set_must_match_metadata(tmp_path):
    """A refined weight saved without its offsets: the loader then expects an
    unrefined weight and finds a mask it has no buffer for."""
    import dataclasses
    t = dataclasses.replace(_random_packed(*CASES[1][1:], seed=3), offsets=None)
    path = tmp_path / "partial.safetensors"
    A.save_packed(path, {"w": t})
    with pytest.raises(ValueError, match="unexpected"):
        A.load_packed(path, device="cpu")


def test_names_with_dots_are_refused(tmp_path):
    t = _random_packed(*CASES[0][1:], seed=1)
    with pytest.raises(ValueError):
        A.save_packed(tmp_path / "x.safetensors", {"layer.0": t})
