"""The C ABI library loads, exports every declared symbol and rejects bad
arguments before launching anything (CPU only: no kernel runs here)."""

import ctypes as C
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "autofp.h")
LIB = os.path.join(ROOT, "runtime_mixed_precision_amd", "libautofp.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libautofp.so not built")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(autofp_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_four_operations():
    names = declared()
    for op in ("autofp_quantize", "autofp_gemv", "autofp_gemm", "autofp_policy_signals"):
        assert op in names


def test_every_declared_symbol_is_exported():
    from runtime_mixed_precision_amd import _native as N
    L = N.lib()
    for name in declared():
        assert hasattr(L, name), name
    assert sorted(N.EXPORTS) == declared()
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (autofp_\w+)", out))
    assert set(declared()) <= exported
    assert exported <= set(declared())          # nothing undocumented is exported


@pytest.fixture(scope="module")
def N():
    from runtime_mixed_precision_amd import _native
    _native.lib()
    return _native


def params(N):
    p = N.Params()
    assert N.lib().autofp_default_params(C.byref(p)) == 0
    return p


def test_default_params_are_the_papers(N):
    p = params(N)
    assert p.rho == pytest.approx(0.2) and p.act_nmse_thresh == pytest.approx(0.003)
    assert p.c2 == 2.0 and p.top_k == 10
    assert p.tau == pytest.approx(0.10) and p.lambda_d == pytest.approx(0.7)
    assert (p.alpha, p.beta, p.n_p) == (4, 2, 2)
    assert C.sizeof(N.Params) == 56 and C.sizeof(N.PolicyState) == N.POLICY_STATE_BYTES
    assert N.lib().autofp_default_params(None) == 1


def test_sizes(N):
    L = N.lib()
    out = (C.c_size_t * 5)()
    A6 = N.FMT_AUTOFP6
    assert L.autofp_packed_bytes(16, 256, N.ACTIVATION, A6, 1, 0, out) == 0
    assert list(out) == [16 * 128, 16 * 16, 4, 16 * 8, 16 * 64]
    assert L.autofp_packed_bytes(256, 4096, N.WEIGHT, A6, 1, 204, out) == 0
    assert list(out) == [256 * 2048, 256 * 256, 4, 128, 256 * 204 + 16]
    assert L.autofp_packed_bytes(16, 250, N.WEIGHT, A6, 0, 0, out) == 2
    # the variant formats: AutoFP6E stores as AutoFP6; AutoFP8 two offset
    # bytes per subgroup; FP6G 3k/4 code bytes and no refinement
    assert L.autofp_packed_bytes(256, 4096, N.WEIGHT, N.FMT_AUTOFP6E, 1, 204, out) == 0
    assert list(out) == [256 * 2048, 256 * 256, 4, 128, 256 * 204 + 16]
    assert L.autofp_packed_bytes(256, 4096, N.WEIGHT, N.FMT_AUTOFP8, 1, 204, out) == 0
    assert list(out) == [256 * 2048, 256 * 256, 4, 128, 2 * 256 * 204 + 16]
    assert L.autofp_packed_bytes(16, 256, N.ACTIVATION, N.FMT_AUTOFP8, 1, 0, out) == 0
    assert list(out) == [16 * 128, 16 * 16, 4, 16 * 8, 16 * 128]
    assert L.autofp_packed_bytes(16, 256, N.ACTIVATION, N.FMT_FP6G, 0, 0, out) == 0
    assert list(out) == [16 * 192, 16 * 16, 4, 0, 0]
    assert L.autofp_packed_bytes(16, 256, N.ACTIVATION, N.FMT_FP6G, 1, 0, out) == 8
    assert L.autofp_packed_bytes(16, 256, N.ACTIVATION, 4, 0, 0, out) == 8
    n = C.c_int32()
    p = params(N)
    for k, want in ((4096, 204), (14336, 716), (256, 12), (16, 0)):
        assert L.autofp_weight_refined_count(k, C.byref(p), C.byref(n)) == 0
        assert n.value == want
    p.rho = 1.0                        # capped at two refined subgroups per group
    assert L.autofp_weight_refined_count(256, C.byref(p), C.byref(n)) == 0 and n.value == 32
    p.rho = 1.5
    assert L.autofp_weight_refined_count(256, C.byref(p), C.byref(n)) == 8
    b = C.c_size_t()
    for op in (N.OP_QUANTIZE, N.OP_SELECT_MASK, N.OP_GEMV, N.OP_GEMM):
        assert L.autofp_workspace_bytes(op, 64, 4096, C.byref(b)) == 0 and b.value > 0
    assert L.autofp_workspace_bytes(9, 64, 4096, C.byref(b)) == 8
    assert L.autofp_workspace_bytes(N.OP_GEMV, 0, 4096, C.byref(b)) == 2
    assert L.autofp_status_string(5) == b"workspace missing or too small"


FAKE = 0x10000    # aligned, never dereferenced: every call below fails its checks first


def packed(N, kind, rows=4, k=64, refine=False, n_refined=0):
    p = N.Packed(rows, k, kind, n_refined, FAKE, FAKE, FAKE, None, None)
    if refine:
        p.mask = FAKE
        p.offsets = FAKE
    return p


def test_quantize_rejects_bad_arguments(N):
    L = N.lib()
    p = params(N)
    ws = C.c_void_p(FAKE)
    q = lambda x, dt, ref, out, wsz=1 << 20: L.autofp_quantize(x, dt, ref, None, C.byref(p), out, ws, wsz, None)
    good = packed(N, N.ACTIVATION)
    assert q(None, N.F32, 0, C.byref(good)) == 1
    assert q(FAKE, N.F32, 0, None) == 1
    assert q(FAKE, 7, 0, C.byref(good)) == 7
    bad = packed(N, N.ACTIVATION, k=40)
    assert q(FAKE, N.F32, 0, C.byref(bad)) == 2
    bad = packed(N, 5)
    assert q(FAKE, N.F32, 0, C.byref(bad)) == 4
    assert q(FAKE, N.F32, 1, C.byref(good)) == 6          # refine without mask/offsets
    assert q(FAKE + 4, N.F32, 0, C.byref(good)) == 8      # misaligned input
    assert q(FAKE, N.F32, 0, C.byref(good), 8) == 5       # workspace too small
    fmt = packed(N, N.ACTIVATION)
    fmt.format = 4
    assert q(FAKE, N.F32, 0, C.byref(fmt)) == 8           # unknown format
    fmt = packed(N, N.ACTIVATION, refine=True)
    fmt.format = N.FMT_FP6G
    assert q(FAKE, N.F32, 1, C.byref(fmt)) == 8           # FP6G has no refinement


def test_quantize_noalloc_checks_and_size_limit(N):
    """The static-scratch encode checks its arguments like autofp_quantize and
    rejects any k whose scratch would pass 64 KiB (k > 491488) before touching
    the device."""
    L = N.lib()
    p = params(N)
    q = lambda x, dt, ref, out: L.autofp_quantize_noalloc(x, dt, ref, None, C.byref(p), out, None)
    good = packed(N, N.ACTIVATION)
    assert q(None, N.F32, 0, C.byref(good)) == 1
    assert q(FAKE, 7, 0, C.byref(good)) == 7
    assert q(FAKE, N.F32, 1, C.byref(good)) == 6
    assert q(FAKE, N.F32, 0, C.byref(packed(N, N.ACTIVATION, k=40))) == 2
    assert q(FAKE, N.F32, 0, C.byref(packed(N, N.ACTIVATION, rows=1, k=491504))) == 5
    assert q(FAKE, N.F32, 0, C.byref(packed(N, N.WEIGHT, rows=1, k=491504))) == 5


def test_linear_rejects_bad_arguments(N):
    L = N.lib()
    p = params(N)
    for fn in (L.autofp_gemv, L.autofp_gemm):
        w = packed(N, N.WEIGHT, rows=8, k=64)
        x = packed(N, N.ACTIVATION, rows=2, k=64)
        call = lambda w_, x_, bits, y=FAKE, ws=1 << 20, bd=None: fn(
            C.byref(w_), C.byref(x_), bits, bd, y, N.F32, C.byref(p), FAKE, ws, None)
        assert call(w, x, 3) == 3                         # level not in {2,4,6}
        assert call(x, w, 4) == 4                         # swapped operands
        assert call(w, x, 6) == 6                         # level 6 without refinement
        assert call(w, x, 4, bd=FAKE) == 6                # device level needs refinement
        assert call(w, x, 4, y=None) == 1
        assert call(w, x, 4, ws=16) == 5
        x2 = packed(N, N.ACTIVATION, rows=2, k=128)
        assert call(w, x2, 4) == 2                        # K mismatch
        wbad = packed(N, N.WEIGHT, rows=8, k=64, refine=True, n_refined=99)
        assert call(wbad, x, 4) == 8                      # n_refined beyond 2 per group
        # the largest reduction dimension: 2^22 (one 256-token tile of fp16
        # activation rows stays below 2^31 bytes); one group more is rejected
        kmax = 1 << 22
        wk, xk = packed(N, N.WEIGHT, rows=8, k=kmax + 16), packed(N, N.ACTIVATION, rows=2, k=kmax + 16)
        assert call(wk, xk, 4) == 2
        wk, xk = packed(N, N.WEIGHT, rows=8, k=kmax), packed(N, N.ACTIVATION, rows=2, k=kmax)
        assert call(wk, xk, 4, ws=16) == 5                # passes the shape check, fails on workspace
        # formats: both operands alike; level 8 for AutoFP8 only; FP6G at 6 only
        assert call(w, x, 8) == 3
        w8, x8 = packed(N, N.WEIGHT, rows=8, k=64), packed(N, N.ACTIVATION, rows=2, k=64)
        w8.format = N.FMT_AUTOFP8
        assert call(w8, x, 4) == 8                        # formats differ
        x8.format = N.FMT_AUTOFP8
        assert call(w8, x8, 8) == 6                       # level 8 needs refinement
        assert call(w8, x8, 4, ws=16) == 5                # level 4 accepted
        wg, xg = packed(N, N.WEIGHT, rows=8, k=64), packed(N, N.ACTIVATION, rows=2, k=64)
        wg.format = xg.format = N.FMT_FP6G
        assert call(wg, xg, 4) == 3 and call(wg, xg, 6, bd=FAKE) == 3
        assert call(wg, xg, 6, ws=16) == 5


def test_gptq_rejects_bad_arguments(N):
    L = N.lib()
    p = params(N)
    g = lambda w, rows, k, out, ws=1 << 30: L.autofp_gptq_quantize(w, rows, k, FAKE, FAKE, C.byref(p), out, FAKE,
                                                                   ws, None)
    good = packed(N, N.WEIGHT, rows=4, k=64, refine=True, n_refined=3)
    assert g(None, 4, 64, C.byref(good)) == 1
    assert g(FAKE, 4, 40, C.byref(good)) == 2                 # k % 16
    assert g(FAKE, 5, 64, C.byref(good)) == 2                 # rows differ from the output's
    assert g(FAKE, 4, 64, C.byref(packed(N, N.ACTIVATION, rows=4, k=64))) == 4
    assert g(FAKE, 4, 64, C.byref(packed(N, N.WEIGHT, rows=4, k=64))) == 6   # no mask / offsets
    bad = packed(N, N.WEIGHT, rows=4, k=64, refine=True, n_refined=2)
    assert g(FAKE, 4, 64, C.byref(bad)) == 8                  # n_refined is not the budget
    bad = packed(N, N.WEIGHT, rows=4, k=64, refine=True, n_refined=3)
    bad.format = N.FMT_AUTOFP8
    assert g(FAKE, 4, 64, C.byref(bad)) == 8
    assert g(FAKE, 4, 64, C.byref(good), ws=16) == 5
    assert g(FAKE + 8, 4, 64, C.byref(good)) == 8             # misaligned weight
    b = C.c_size_t()
    assert L.autofp_workspace_bytes(N.OP_GPTQ, 4096, 4096, C.byref(b)) == 0 and b.value > 10 * 4096 * 4096
    assert L.autofp_workspace_bytes(N.OP_GPTQ, 8, 65552, C.byref(b)) == 2


def test_signals_reject_bad_arguments(N):
    L = N.lib()
    p = params(N)
    sig = lambda *a, ws=FAKE, wsb=1 << 30: L.autofp_policy_signals(*a, ws, wsb, None)
    assert sig(FAKE, 1, 100, None, None, N.F32, 0, C.byref(p), None, None) == 1
    assert sig(None, 1, 100, None, None, N.F32, 0, C.byref(p), FAKE, None) == 1
    p.top_k = 40
    assert sig(FAKE, 1, 100, None, None, N.F32, 0, C.byref(p), FAKE, None) == 8
    p.top_k = 10
    assert sig(None, 1, 0, FAKE, FAKE, 3, 64, C.byref(p), None, FAKE) == 7
    assert sig(None, 0, 0, FAKE, FAKE, N.F32, 64, C.byref(p), None, FAKE) == 2
    # G_E needs the slice workspace; L_A alone does not
    need = C.c_size_t()
    assert L.autofp_workspace_bytes(N.OP_SIGNALS, 2, 128256, C.byref(need)) == 0
    assert sig(FAKE, 2, 128256, None, None, N.F32, 0, C.byref(p), FAKE, None, ws=None) == 5
    assert sig(FAKE, 2, 128256, None, None, N.F32, 0, C.byref(p), FAKE, None, wsb=need.value - 1) == 5
    assert sig(FAKE, 70000, 100, None, None, N.F32, 0, C.byref(p), FAKE, None) == 2


def test_signals_workspace_size(N):
    L = N.lib()
    b = C.c_size_t()
    # one candidate list of up to 32 floats per 4096-logit slice
    for batch, vocab in ((1, 128256), (64, 128256), (3, 50257), (1, 1)):
        assert L.autofp_workspace_bytes(N.OP_SIGNALS, batch, vocab, C.byref(b)) == 0
        slices = -(-vocab // 4096)
        assert b.value >= batch * slices * 32 * 4
    assert L.autofp_workspace_bytes(N.OP_SIGNALS, 0, 100, C.byref(b)) == 2
    assert L.autofp_workspace_bytes(N.OP_SIGNALS, 1, 0, C.byref(b)) == 2


def test_policy_update_rejects_bad_arguments(N):
    L = N.lib()
    p = params(N)
    up = lambda phase, layer, la, ge, batch, st, br: L.autofp_policy_update(
        phase, layer, 0, la, ge, batch, C.byref(p), st, br, None, None)
    assert up(0, 0, None, None, 1, FAKE, FAKE) == 1
    assert up(1, 0, FAKE, None, 1, FAKE, FAKE) == 1        # decode needs G_E
    assert up(2, 0, FAKE, FAKE, 1, FAKE, FAKE) == 8
    assert up(0, -1, FAKE, FAKE, 1, FAKE, FAKE) == 8
    assert up(0, 0, FAKE, FAKE, 0, FAKE, FAKE) == 2
    p.alpha = 0
    assert up(1, 0, FAKE, FAKE, 1, FAKE, FAKE) == 8


def test_policy_layer_rejects_bad_arguments(N):
    L = N.lib()
    p = params(N)
    pl = lambda phase, layer, hp, hc, dt, hidden, ge, batch, st, la, br: L.autofp_policy_layer(
        phase, layer, 0, hp, hc, dt, hidden, ge, batch, C.byref(p), st, la, br, None, None)
    assert pl(0, 0, None, FAKE, N.F32, 16, None, 1, FAKE, FAKE, FAKE) == 1
    assert pl(0, 0, FAKE, FAKE, N.F32, 16, None, 1, FAKE, None, FAKE) == 1   # l_a output
    assert pl(1, 0, FAKE, FAKE, N.F32, 16, None, 1, FAKE, FAKE, FAKE) == 1   # decode needs G_E
    assert pl(2, 0, FAKE, FAKE, N.F32, 16, FAKE, 1, FAKE, FAKE, FAKE) == 8
    assert pl(0, 0, FAKE, FAKE, N.F32, 0, None, 1, FAKE, FAKE, FAKE) == 2
    assert pl(0, 0, FAKE, FAKE, N.F32, 16, None, 0, FAKE, FAKE, FAKE) == 2
    assert pl(0, 0, FAKE, FAKE, 9, 16, None, 1, FAKE, FAKE, FAKE) == 7   # dtype
    p.alpha = 0
    assert pl(0, 1, FAKE, FAKE, N.F32, 16, None, 1, FAKE, FAKE, FAKE) == 8


def kv_cache(N, h_kv=8, n_pages=4, max_pages=4, head_dim=128):
    return N.KvCache(h_kv, head_dim, n_pages, max_pages, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_kv_workspace_sizes(N):
    L = N.lib()
    b = C.c_size_t()
    assert C.sizeof(N.KvCache) == 80
    assert L.autofp_workspace_bytes(N.OP_KV_WRITE, 16, 128, C.byref(b)) == 0 and b.value >= 2 * 4 * 1024
    assert L.autofp_workspace_bytes(N.OP_KV_WRITE, 16, 64, C.byref(b)) == 2
    # one record of 128 + 4 floats per (row, context split)
    assert L.autofp_workspace_bytes(N.OP_KV_ATTENTION, 512, 512, C.byref(b)) == 0
    assert b.value % (512 * 132 * 4) == 0 and 1 <= b.value // (512 * 132 * 4) <= 64
    assert L.autofp_workspace_bytes(N.OP_KV_ATTENTION, 1, 1, C.byref(b)) == 0 and b.value == 132 * 4
    assert L.autofp_workspace_bytes(N.OP_KV_ATTENTION, 4, 64 * 64 + 1, C.byref(b)) == 2


def test_kv_write_rejects_bad_arguments(N):
    L = N.lib()
    c = kv_cache(N)
    w = lambda k, v, dt, n, slots, c_, ws=FAKE, wsb=1 << 20, ss=0: L.autofp_kv_write(
        k, v, dt, n, slots, ss, c_, ws, wsb, None)
    assert w(None, FAKE, N.F32, 4, FAKE, C.byref(c)) == 1
    assert w(FAKE, FAKE, N.F32, 4, None, C.byref(c)) == 1
    assert w(FAKE, FAKE, N.F32, 4, FAKE, None) == 1
    assert w(FAKE, FAKE, 3, 4, FAKE, C.byref(c)) == 7
    assert w(FAKE, FAKE, N.F32, 0, FAKE, C.byref(c)) == 2
    bad = kv_cache(N, head_dim=64)
    assert w(FAKE, FAKE, N.F32, 4, FAKE, C.byref(bad)) == 2
    assert w(FAKE + 4, FAKE, N.F32, 4, FAKE, C.byref(c)) == 8
    assert w(FAKE, FAKE, N.F32, 4, FAKE, C.byref(c), ws=None, ss=1) == 5   # the scale pass needs scratch
    assert w(FAKE, FAKE, N.F32, 4, FAKE, C.byref(c), wsb=16, ss=1) == 5


def test_kv_attention_rejects_bad_arguments(N):
    L = N.lib()
    c = kv_cache(N)
    a = lambda q, batch, hq, c_, bits=4, out=FAKE, ws=FAKE, wsb=1 << 30, dt=0, sm=0.088: \
        L.autofp_kv_attention(q, dt, batch, hq, c_, bits, None, sm, out, ws, wsb, None)
    assert a(None, 2, 32, C.byref(c)) == 1
    assert a(FAKE, 2, 32, C.byref(c), out=None) == 1
    assert a(FAKE, 2, 30, C.byref(c)) == 2                 # 30 query heads over 8 KV heads
    assert a(FAKE, 2, 8 * 17, C.byref(c)) == 2             # more than 16 query heads per KV head
    assert a(FAKE, 0, 32, C.byref(c)) == 2
    assert a(FAKE, 2, 32, C.byref(c), bits=5) == 3
    assert a(FAKE, 2, 32, C.byref(c), dt=4) == 7
    assert a(FAKE, 2, 32, C.byref(c), sm=float("inf")) == 8
    assert a(FAKE, 2, 32, C.byref(c), wsb=16) == 5
    assert a(FAKE, 2, 32, C.byref(c), ws=None) == 5
    nt = kv_cache(N)
    nt.page_table = None
    assert a(FAKE, 2, 32, C.byref(nt)) == 1
    big = kv_cache(N, max_pages=64 * 64 + 1)
    assert a(FAKE, 2, 32, C.byref(big)) == 2


def test_epilogue_rejects_bad_arguments_and_sizes_its_workspace(N):
    """autofp_epilogue_quantize's checks (no launch is reached): unknown op,
    a residual op without its residual, z narrower than k, and a workspace
    of autofp_quantize's size for RESIDUAL_RMSNORM, which needs one more fp32
    per row (AUTOFP_OP_EPILOGUE)."""
    L = N.lib()
    p = params(N)
    rows, k = 4, 64
    wq, we = C.c_size_t(), C.c_size_t()
    assert L.autofp_workspace_bytes(N.OP_QUANTIZE, rows, k, C.byref(wq)) == 0
    assert L.autofp_workspace_bytes(N.OP_EPILOGUE, rows, k, C.byref(we)) == 0
    assert we.value >= wq.value + 4 * rows
    out = packed(N, N.ACTIVATION, rows=rows, k=k)
    e = lambda op, resid, ldz, wsz: L.autofp_epilogue_quantize(op, FAKE, ldz, resid, None, 0, None, C.byref(p),
                                                               C.byref(out), FAKE, wsz, None)
    big = we.value
    assert e(5, FAKE, k, big) == 8                                  # unknown op
    assert e(N.EPI_RESIDUAL_RMSNORM, None, k, big) == 1             # residual missing
    assert e(N.EPI_RESIDUAL, None, k, big) == 1
    assert e(N.EPI_RESIDUAL_RMSNORM, FAKE, k - 4, big) == 2         # ldz < k
    assert e(N.EPI_RESIDUAL_RMSNORM, FAKE, k, wq.value) == 5        # the encode's workspace is short


def test_layer_epilogue_rejects_bad_arguments(N):
    """autofp_layer_epilogue's checks (no launch is reached): the required
    pointers, the policy arguments (phase, decode without g_e), v_out equal to
    h_prev or to the residual, z narrower than k, a workspace of the
    encode's size (AUTOFP_OP_EPILOGUE needs one more fp32 per row)."""
    L = N.lib()
    p = params(N)
    rows, k = 2, 64
    wq, we = C.c_size_t(), C.c_size_t()
    assert L.autofp_workspace_bytes(N.OP_QUANTIZE, rows, k, C.byref(wq)) == 0
    assert L.autofp_workspace_bytes(N.OP_EPILOGUE, rows, k, C.byref(we)) == 0
    out = packed(N, N.ACTIVATION, rows=rows, k=k)
    F2, F3, F4 = FAKE + 4096, FAKE + 8192, FAKE + 12288

    def e(z=FAKE, ldz=k, resid=F2, v_out=F3, h_prev=F4, phase=1, g_e=FAKE, state=FAKE, l_a=FAKE, bits=FAKE,
          wsz=None):
        return L.autofp_layer_epilogue(z, ldz, resid, v_out, h_prev, 0, None, phase, 0, 0, g_e, C.byref(p),
                                       state, l_a, bits, None, C.byref(out), FAKE,
                                       we.value if wsz is None else wsz, None)
    for kw in ("z", "resid", "v_out", "h_prev", "state", "l_a", "bits"):
        assert e(**{kw: None}) == 1, kw                    # AUTOFP_ERR_NULL
    assert e(g_e=None) == 1                                # decode needs G_E
    assert e(phase=2) == 8                                 # AUTOFP_ERR_ARG
    assert e(v_out=F4) == 8                                # v_out is h_prev
    assert e(v_out=F2) == 8                                # v_out is the residual
    assert e(ldz=k - 4) == 2                               # AUTOFP_ERR_SHAPE
    assert e(wsz=wq.value) == 5                            # AUTOFP_ERR_WORKSPACE
