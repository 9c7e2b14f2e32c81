"""Host-side logic that needs no GPU: the benchmark's byte accounting and its
one-GPU guard, and the KV page plan that the KV tests and the benchmark use
to lay tokens out over base and refinement pages."""

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from runtime_mixed_precision_amd import synthetic as S  # noqa: E402


def fake_packed(rows, k, refine):
    """Byte counts of a packed weight laid out as the C ABI describes: codes
    k/2 and E4M3 scales k/16 per row; the shared mask k/32 and R = floor(0.2 k/4)
    offset bytes per row (+ 16 pad bytes) at level 6."""
    r = int(0.2 * k / 4)
    t = lambda n: SimpleNamespace(numel=lambda: n)
    return SimpleNamespace(rows=rows, k=k, codes=t(rows * k // 2), scales=t(rows * k // 16),
                           mask=t((k + 31) // 32) if refine else t(0),
                           offsets=t(rows * r + 16) if refine else t(0))


@pytest.mark.parametrize("name,rows,k,b4", [("wqkv", 6144, 4096, 14155780), ("wo", 4096, 4096, 9437188),
                                            ("wdown", 4096, 14336, 33030148)])
def test_weight_bytes_closed_form(name, rows, k, b4):
    """4.5 bits per weight plus the 4-byte tensor scale at levels 2 and 4;
    level 6 adds R bytes per row and the mask (4.9 bits at rho = 0.2)."""
    wp = fake_packed(rows, k, True)
    assert bench.w_bytes(wp, 4) == b4 == bench.w_bytes(wp, 2)
    r = int(0.2 * k / 4)
    assert bench.w_bytes(wp, 6) == b4 + k // 32 + rows * r + 16
    bits6 = 8 * (bench.w_bytes(wp, 6) - 4) / (rows * k)
    assert abs(bits6 - 4.9) < 0.01


def test_activation_and_gemv_bytes():
    # one token of 4096: 2048 code bytes + 256 scales + T; level 6 adds the
    # mask (128 B) and the dense offsets (1024 B)
    assert bench.x_bytes(1, 4096, 4) == 2048 + 256 + 4
    assert bench.x_bytes(1, 4096, 6) == 2048 + 256 + 4 + 128 + 1024
    wp = fake_packed(4096, 4096, False)
    assert bench.gemv_bytes(wp, 8, 4) == bench.w_bytes(wp, 4) + bench.x_bytes(8, 4096, 4) + 4 * 8 * 4096
    assert bench.encode_bytes(8, 4096, 4) == 2 * 8 * 4096 + bench.x_bytes(8, 4096, 4)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("frac", [0.0, 0.3, 1.0])
def test_kv_page_plan_invariants(frac):
    lengths = [0, 1, 63, 64, 65, 300, 1000]
    plan = S.kv_page_plan(lengths, frac, seed=3)
    kind, fill, table = plan["page_kind"], plan["page_tokens"], plan["page_table"]
    n_pages = plan["n_pages"]
    used = np.zeros(n_pages, np.int64)
    all_slots = []
    for b, L in enumerate(lengths):
        slots = np.asarray(plan["slots"][b], np.int64)
        ref = np.asarray(plan["refine"][b], bool)
        assert len(slots) == L and len(ref) == L
        pages, pos = slots // 64, slots % 64
        # a refinement page holds refined tokens only, at most 32; a base page up to 64
        assert np.all(kind[pages] == ref.astype(np.uint8))
        assert np.all(pos < np.where(ref, 32, 64))
        np.add.at(used, pages, 1)
        # the sequence's page list is exactly the pages its tokens use
        listed = table[b, :plan["seq_pages"][b]]
        assert set(listed.tolist()) == set(pages.tolist())
        assert np.all(table[b, plan["seq_pages"][b]:] == -1)
        all_slots.append(slots)
    all_slots = np.concatenate(all_slots) if all_slots else np.zeros(0, np.int64)
    assert len(np.unique(all_slots)) == len(all_slots)          # no slot written twice
    assert np.array_equal(used[:len(fill)], fill.astype(np.int64))
    if frac == 0.0:
        assert not kind.any()
    if frac == 1.0:
        assert kind[fill > 0].all()


def test_kv_tokens_are_seeded():
    a = S.kv_tokens(5, 2, seed=7, tensor_id=1)
    b = S.kv_tokens(5, 2, seed=7, tensor_id=1)
    c = S.kv_tokens(5, 2, seed=7, tensor_id=2)
    assert a.dtype == torch.bfloat16 and a.shape == (5, 2, 128)
    assert torch.equal(a, b) and not torch.equal(a, c)
