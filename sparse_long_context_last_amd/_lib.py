"""ctypes declarations of the C ABI in include/fp_prefill.h (argument
marshalling only; every computation happens in libfp_prefill.so)."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp_prefill.so")

FP_OK = 0
FP_ERR_INVALID_ARG = -1
FP_ERR_UNSUPPORTED = -2
FP_ERR_SHAPE = -3
FP_ERR_OOM = -4
FP_ERR_HIP = -5
FP_BF16 = 0
FP_FP32 = 1
FP_PATTERN_VERTICAL_SLASH = 0
FP_PATTERN_QUERY_AWARE = 1
FP_LAYOUT_BHND = 0
FP_LAYOUT_THD = 1
DEBUG_ITEMS = {"qbar": 0, "kbar": 1, "rowmax": 2, "rowsum": 3, "colsum": 4,
               "diagsum": 5, "atrue": 6, "ahat": 7, "counts": 8,
               "colptr": 9, "colidx": 10}


class PlanInfo(C.Structure):
    _fields_ = [("B", C.c_int), ("Hq", C.c_int), ("Hkv", C.c_int), ("N", C.c_int),
                ("d", C.c_int), ("block", C.c_int), ("nb", C.c_int), ("dtype", C.c_int),
                ("gamma", C.c_float), ("tau", C.c_float), ("min_budget", C.c_int),
                ("total_blocks", C.c_longlong), ("dense_blocks", C.c_longlong),
                ("query_aware_heads", C.c_int), ("max_budget", C.c_int),
                ("qa_selection", C.c_int), ("layout", C.c_int), ("vs_granularity", C.c_int),
                ("tokens", C.c_longlong), ("rows", C.c_longlong)]


class PlanOptions(C.Structure):
    _fields_ = [("max_budget", C.c_int), ("qa_selection", C.c_int), ("vs_granularity", C.c_int)]


QA_SELECTION = {"flattened": 0, "querywise": 1}
VS_GRANULARITY = {"block": 0, "token": 1}


# name -> (restype, argtypes)
SIGNATURES = {
    "fp_prefill_plan": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int,
                                  C.c_int, C.c_int, C.c_int, C.c_float, C.c_float, C.c_int,
                                  C.c_void_p, C.POINTER(C.c_void_p)]),
    "fp_prefill_plan_ex": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int,
                                     C.c_int, C.c_int, C.c_int, C.c_float, C.c_float, C.c_int,
                                     C.POINTER(PlanOptions), C.c_void_p, C.POINTER(C.c_void_p)]),
    "fp_prefill_plan_varlen": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                         C.c_int, C.c_int, C.c_int, C.c_float, C.c_float, C.c_int,
                                         C.POINTER(PlanOptions), C.c_void_p, C.POINTER(C.c_void_p)]),
    "fp_prefill_attend": (C.c_int, [C.c_void_p] * 6),
    "fp_prefill_attend_noalloc": (C.c_int, [C.c_void_p] * 6),
    "fp_dense_attend": (C.c_int, [C.c_void_p] * 4 + [C.c_int] * 7 + [C.c_void_p]),
    "fp_dense_attend_varlen": (C.c_int, [C.c_void_p] * 4 + [C.c_int, C.c_int, C.c_void_p] + [C.c_int] * 4
                               + [C.c_void_p]),
    "fp_plan_info_get": (C.c_int, [C.c_void_p, C.POINTER(PlanInfo)]),
    "fp_plan_copy_out": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p]),
    "fp_plan_copy_debug": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_size_t]),
    "fp_plan_destroy": (None, [C.c_void_p]),
    "fp_workspace_trim": (C.c_int, []),
    "fp_status_str": (C.c_char_p, [C.c_int]),
    "fp_last_error": (C.c_char_p, []),
    "fp_profile_enable": (C.c_int, [C.c_int]),
    "fp_profile_read": (C.c_int, [C.POINTER(C.c_double), C.POINTER(C.c_longlong),
                                  C.POINTER(C.c_double), C.POINTER(C.c_longlong), C.c_int]),
    "fp_canonical_constants": (C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p]),
    "fp_probe_exp2": (C.c_int, [C.c_void_p, C.c_void_p, C.c_longlong, C.c_void_p]),
    "fp_probe_ln": (C.c_int, [C.c_void_p, C.c_void_p, C.c_longlong, C.c_void_p]),
    "fp_probe_sqrt": (C.c_int, [C.c_void_p, C.c_void_p, C.c_longlong, C.c_void_p]),
}

_lib = None


def load() -> C.CDLL:
    """Load libfp_prefill.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_long_context_last_amd.build` "
            "(there is no fallback implementation)")
    # torch ships its own HIP runtime; it must be the one this library binds
    # to (a second runtime in the same process does not see the device), so
    # torch is imported first and the library's libamdhip64 dependency then
    # resolves to the copy torch already loaded.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FpError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        msg = lib.fp_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.fp_status_str(status).decode()} ({msg})")


def check(status: int, where: str) -> None:
    if status != FP_OK:
        raise FpError(status, where)
