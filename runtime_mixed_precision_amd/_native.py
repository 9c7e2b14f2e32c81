"""ctypes view of libautofp.so (the C ABI of include/autofp.h).

The library is loaded on first use; a missing or unloadable library raises
``NativeLibraryError`` - there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("AUTOFP_LIB", os.path.join(PKG, "libautofp.so"))

OK = 0
STATUS_NAMES = {
    0: "AUTOFP_OK", 1: "AUTOFP_ERR_NULL", 2: "AUTOFP_ERR_SHAPE", 3: "AUTOFP_ERR_BITS",
    4: "AUTOFP_ERR_KIND", 5: "AUTOFP_ERR_WORKSPACE", 6: "AUTOFP_ERR_MISSING_REFINEMENT",
    7: "AUTOFP_ERR_DTYPE", 8: "AUTOFP_ERR_ARG", 9: "AUTOFP_ERR_HIP",
}
F32, BF16 = 0, 1
WEIGHT, ACTIVATION = 0, 1
OP_QUANTIZE, OP_SELECT_MASK, OP_GEMV, OP_GEMM, OP_SIGNALS = 0, 1, 2, 3, 4
OP_KV_WRITE, OP_KV_ATTENTION, OP_GPTQ, OP_EPILOGUE = 5, 6, 7, 8
KV_PAGE_TOKENS, KV_HEAD_DIM, KV_PAGE_BYTES = 64, 128, 4608
EPI_COPY, EPI_RESIDUAL, EPI_SWIGLU, EPI_RESIDUAL_RMSNORM = 1, 2, 3, 4
FMT_AUTOFP6, FMT_AUTOFP6E, FMT_AUTOFP8, FMT_FP6G = 0, 1, 2, 3
FORMATS = {"autofp6": FMT_AUTOFP6, "autofp6e": FMT_AUTOFP6E, "autofp8": FMT_AUTOFP8, "fp6g": FMT_FP6G}

# Every symbol include/autofp.h declares.
EXPORTS = (
    "autofp_default_params", "autofp_status_string", "autofp_packed_bytes",
    "autofp_weight_refined_count", "autofp_workspace_bytes", "autofp_select_weight_mask",
    "autofp_quantize", "autofp_quantize_noalloc", "autofp_gptq_quantize", "autofp_epilogue_quantize",
    "autofp_layer_epilogue", "autofp_gemv", "autofp_gemv_rows", "autofp_gemm", "autofp_policy_signals",
    "autofp_policy_update", "autofp_policy_layer", "autofp_kv_write", "autofp_kv_attention",
)


class NativeLibraryError(RuntimeError):
    pass


class AutofpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


class Params(C.Structure):
    _fields_ = [("rho", C.c_double), ("act_nmse_thresh", C.c_float), ("c2", C.c_float),
                ("top_k", C.c_int32), ("eps", C.c_float), ("tau", C.c_double),
                ("lambda_d", C.c_double), ("alpha", C.c_int32), ("beta", C.c_int32),
                ("n_p", C.c_int32), ("gemv_waves", C.c_int32)]


class PolicyState(C.Structure):
    _fields_ = [("mean", C.c_double), ("m2", C.c_double), ("count", C.c_int32), ("up", C.c_int32),
                ("down", C.c_int32), ("bits", C.c_int32), ("spike", C.c_int32),
                ("reserved", C.c_int32 * 3)]


POLICY_STATE_BYTES = 48


class Packed(C.Structure):
    _fields_ = [("rows", C.c_int64), ("k", C.c_int64), ("kind", C.c_int32), ("n_refined", C.c_int32),
                ("codes", C.c_void_p), ("scales", C.c_void_p), ("tensor_scale", C.c_void_p),
                ("mask", C.c_void_p), ("offsets", C.c_void_p), ("format", C.c_int32), ("reserved", C.c_int32)]


class KvCache(C.Structure):
    _fields_ = [("h_kv", C.c_int32), ("head_dim", C.c_int32), ("n_pages", C.c_int32),
                ("max_pages", C.c_int32), ("k_pages", C.c_void_p), ("v_pages", C.c_void_p),
                ("page_kind", C.c_void_p), ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("page_table", C.c_void_p), ("seq_pages", C.c_void_p),
                ("page_tokens", C.c_void_p)]


_lib = None


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NativeLibraryError(
            f"{LIB_PATH} is missing: build it with `python -m runtime_mixed_precision_amd.build`")
    try:
        L = C.CDLL(LIB_PATH)
    except OSError as e:
        raise NativeLibraryError(f"cannot load {LIB_PATH}: {e}") from e
    P = C.POINTER
    vp = C.c_void_p
    sig = {
        "autofp_default_params": (C.c_int, [P(Params)]),
        "autofp_status_string": (C.c_char_p, [C.c_int]),
        "autofp_packed_bytes": (C.c_int, [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                          P(C.c_size_t)]),
        "autofp_weight_refined_count": (C.c_int, [C.c_int64, P(Params), P(C.c_int32)]),
        "autofp_workspace_bytes": (C.c_int, [C.c_int32, C.c_int64, C.c_int64, P(C.c_size_t)]),
        "autofp_select_weight_mask": (C.c_int, [vp, C.c_int64, C.c_int64, C.c_int32, P(Params), vp, vp,
                                                C.c_size_t, vp]),
        "autofp_quantize": (C.c_int, [vp, C.c_int32, C.c_int32, vp, P(Params), P(Packed), vp,
                                      C.c_size_t, vp]),
        "autofp_quantize_noalloc": (C.c_int, [vp, C.c_int32, C.c_int32, vp, P(Params), P(Packed), vp]),
        "autofp_gptq_quantize": (C.c_int, [vp, C.c_int64, C.c_int64, vp, vp, P(Params), P(Packed), vp, C.c_size_t, vp]),
        "autofp_epilogue_quantize": (C.c_int, [C.c_int32, vp, C.c_int64, vp, vp, C.c_int32, vp, P(Params),
                                               P(Packed), vp, C.c_size_t, vp]),
        "autofp_layer_epilogue": (C.c_int, [vp, C.c_int64, vp, vp, vp, C.c_int32, vp, C.c_int32, C.c_int32,
                                            C.c_int32, vp, P(Params), vp, vp, vp, vp, P(Packed), vp,
                                            C.c_size_t, vp]),
        "autofp_gemv": (C.c_int, [P(Packed), P(Packed), C.c_int32, vp, vp, C.c_int32, P(Params), vp,
                                  C.c_size_t, vp]),
        "autofp_gemv_rows": (C.c_int, [P(Packed), P(Packed), vp, vp, C.c_int32, P(Params), vp, C.c_size_t, vp]),
        "autofp_gemm": (C.c_int, [P(Packed), P(Packed), C.c_int32, vp, vp, C.c_int32, P(Params), vp,
                                  C.c_size_t, vp]),
        "autofp_policy_signals": (C.c_int, [vp, C.c_int64, C.c_int64, vp, vp, C.c_int32, C.c_int64,
                                            P(Params), vp, vp, vp, C.c_size_t, vp]),
        "autofp_policy_update": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, vp, vp, C.c_int64,
                                           P(Params), vp, vp, vp, vp]),
        "autofp_policy_layer": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, vp, vp, C.c_int32, C.c_int64, vp,
                                          C.c_int64, P(Params), vp, vp, vp, vp, vp]),
        "autofp_kv_write": (C.c_int, [vp, vp, C.c_int32, C.c_int64, vp, C.c_int32, P(KvCache), vp,
                                      C.c_size_t, vp]),
        "autofp_kv_attention": (C.c_int, [vp, C.c_int32, C.c_int64, C.c_int32, P(KvCache), C.c_int32,
                                          vp, C.c_float, vp, vp, C.c_size_t, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def check(status, where):
    if status != OK:
        raise AutofpError(status, where)
