"""The C-ABI library loads, exports every symbol include/fp_prefill.h
declares, and validates arguments on the host (no GPU needed: every call here
fails validation or is an empty problem before any HIP call)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp_prefill.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_long_context_last_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_long_context_last_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp_prefill_plan", "fp_prefill_attend", "fp_dense_attend", "fp_plan_info_get",
              "fp_plan_copy_out", "fp_plan_destroy", "fp_status_str", "fp_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from sparse_long_context_last_amd import _lib
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings(lib):
    for code, name in [(0, "FP_OK"), (-1, "FP_ERR_INVALID_ARG"), (-2, "FP_ERR_UNSUPPORTED"),
                       (-3, "FP_ERR_SHAPE"), (-4, "FP_ERR_OOM"), (-5, "FP_ERR_HIP")]:
        assert lib.fp_status_str(code).decode() == name


def _plan(lib, dtype=0, B=1, Hq=4, Hkv=4, N=1024, d=128, block=128, gamma=0.95, tau=0.1,
          min_budget=1024, q=1, k=1, out=True):
    h = C.c_void_p()
    st = lib.fp_prefill_plan(q, k, dtype, B, Hq, Hkv, N, d, block, gamma, tau, min_budget, None,
                             C.byref(h) if out else None)
    return st, h


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(d=32), -2), (dict(d=256), -2), (dict(block=32), -2), (dict(dtype=7), -2),
    (dict(Hq=6, Hkv=4), -3), (dict(N=128 * 4097), -3), (dict(N=128 * 4096 + 1), -3), (dict(Hkv=0), -3),
    (dict(gamma=0.0), -1), (dict(gamma=1.5), -1), (dict(gamma=float("nan")), -1),
    (dict(tau=-0.1), -1), (dict(tau=float("inf")), -1), (dict(min_budget=-1), -1),
    (dict(q=None), -1), (dict(k=None), -1), (dict(B=-1), -1), (dict(out=False), -1),
])
def test_plan_validation(lib, kw, code):
    st, h = _plan(lib, **kw)
    assert st == code, lib.fp_last_error()
    assert lib.fp_last_error().decode()
    if kw.get("out", True):
        assert h.value is None


def test_empty_problems_need_no_device(lib):
    from sparse_long_context_last_amd._lib import PlanInfo
    for kw in (dict(B=0), dict(Hq=0), dict(N=0)):
        st, h = _plan(lib, q=None, k=None, **kw)
        assert st == 0, lib.fp_last_error()
        info = PlanInfo()
        assert lib.fp_plan_info_get(h, C.byref(info)) == 0
        assert info.total_blocks == 0 and info.dense_blocks == 0
        rp = np.ones(1, np.int32)
        assert lib.fp_plan_copy_out(h, None, None, rp.ctypes.data, rp.ctypes.data, None) == 0
        assert rp[0] == 0
        assert lib.fp_prefill_attend(h, None, None, None, None, None) == 0
        lib.fp_plan_destroy(h)
    assert lib.fp_dense_attend(None, None, None, None, 0, 0, 4, 4, 1024, 128, 128, None) == 0
    lib.fp_plan_destroy(None)


def test_attend_validation(lib):
    assert lib.fp_prefill_attend(None, 1, 1, 1, 1, None) == -1
    assert lib.fp_dense_attend(1, 1, 1, 1, 0, 1, 4, 4, 1024, 96, 128, None) == -2
    assert lib.fp_dense_attend(1, 1, 1, 1, 0, 1, 4, 3, 1024, 128, 128, None) == -3
    assert lib.fp_dense_attend(None, 1, 1, 1, 0, 1, 4, 4, 1024, 128, 128, None) == -1
    assert lib.fp_plan_copy_debug(None, 0, None, 0) == -1
    assert lib.fp_plan_copy_out(None, None, None, None, None, None) == -1


def test_canonical_constants_match_the_oracle(lib):
    """The library derives its constants on its own (long double on the
    host); they must equal the oracle's (exact rationals) bit for bit."""
    import sparse_long_context_last_amd as F
    for d in (64, 128):
        c = F.canonical_constants(d)
        assert np.array_equal(c["e2"], np.array(O.EXP2_COEF, np.float32))
        assert np.array_equal(c["lnc"], np.array(O.LN_COEF, np.float64))
        assert c["ln2"] == O.LN2_F64 and c["sqrt_half"] == O.SQRT_HALF_F64
        assert c["C"] == O.score_scale(d)


def test_product_path_has_no_fallback():
    """The binding refuses to run without the compiled library."""
    src = open(os.path.join(ROOT, "sparse_long_context_last_amd", "__init__.py")).read()
    src += open(os.path.join(ROOT, "sparse_long_context_last_amd", "_lib.py")).read()
    assert "oracle" not in src and "synth" not in src
    assert "there is no fallback" in src


def test_plan_options_validation(lib):
    from sparse_long_context_last_amd._lib import PlanOptions

    def plan_ex(max_budget=0, qa_selection=0, min_budget=1024, block=128):
        h = C.c_void_p()
        opt = PlanOptions(max_budget, qa_selection)
        return lib.fp_prefill_plan_ex(1, 1, 0, 1, 4, 4, 1024, 128, block, 0.95, 0.1, min_budget, C.byref(opt),
                                      None, C.byref(h))
    assert plan_ex(max_budget=-1) == -1
    assert plan_ex(max_budget=896) == -1          # 7 blocks < the 8 the minimum budget needs
    assert "max_budget" in lib.fp_last_error().decode()
    assert plan_ex(qa_selection=2) == -1
    assert "qa_selection" in lib.fp_last_error().decode()
    assert plan_ex(qa_selection=-1) == -1

    def plan_vs(g):
        h = C.c_void_p()
        opt = PlanOptions(0, 0, g)
        return lib.fp_prefill_plan_ex(1, 1, 0, 1, 4, 4, 1024, 128, 128, 0.95, 0.1, 1024, C.byref(opt),
                                      None, C.byref(h))
    assert plan_vs(2) == -1 and "vs_granularity" in lib.fp_last_error().decode()
    assert plan_vs(-1) == -1
    from sparse_long_context_last_amd._lib import PlanInfo
    for opt in (None, PlanOptions(8192, 1)):
        # valid settings on an empty problem need no device
        h = C.c_void_p()
        assert lib.fp_prefill_plan_ex(None, None, 0, 0, 4, 4, 1024, 128, 128, 0.95, 0.1, 1024,
                                      C.byref(opt) if opt is not None else None, None, C.byref(h)) == 0
        info = PlanInfo()
        assert lib.fp_plan_info_get(h, C.byref(info)) == 0
        assert (info.max_budget, info.qa_selection) == ((8192, 1) if opt is not None else (0, 0))
        lib.fp_plan_destroy(h)


def test_varlen_validation(lib):
    from sparse_long_context_last_amd._lib import PlanInfo

    def plan_v(cu, nseq=None, q=1, Hq=4, Hkv=4, block=128):
        cu = np.asarray(cu, np.int32)
        h = C.c_void_p()
        st = lib.fp_prefill_plan_varlen(q, q, 0, len(cu) - 1 if nseq is None else nseq,
                                        cu.ctypes.data if cu.size else None, Hq, Hkv, 128, block, 0.95, 0.1,
                                        1024, None, None, C.byref(h))
        return st, h
    assert plan_v([1, 5])[0] == -1                        # cu[0] != 0
    assert plan_v([0, 9, 5])[0] == -1                     # decreasing
    assert "decreases" in lib.fp_last_error().decode()
    assert plan_v([], nseq=2)[0] == -1                    # NULL cu_seqlens
    assert plan_v([0, 128 * 4096 + 1])[0] == -3           # more than 4096 blocks
    assert plan_v([0, 100], Hq=6)[0] == -3                # Hq % Hkv
    assert plan_v([0, 100], nseq=-1)[0] == -1
    # no tokens at all: valid, no device needed; every head reports pattern 0
    for cu in ([0], [0, 0, 0]):
        st, h = plan_v(cu, q=None)
        assert st == 0, lib.fp_last_error()
        info = PlanInfo()
        assert lib.fp_plan_info_get(h, C.byref(info)) == 0
        assert info.layout == 1 and info.rows == 0 and info.tokens == 0 and info.total_blocks == 0
        pat = np.ones(max(1, info.B * info.Hq), np.uint8)
        rp = np.ones(1, np.int32)
        assert lib.fp_plan_copy_out(h, pat.ctypes.data, None, rp.ctypes.data, rp.ctypes.data, None) == 0
        assert rp[0] == 0 and (info.B == 0 or not pat.any())
        assert lib.fp_prefill_attend(h, None, None, None, None, None) == 0
        lib.fp_plan_destroy(h)
    cu = np.zeros(3, np.int32)
    assert lib.fp_dense_attend_varlen(None, None, None, None, 0, 2, cu.ctypes.data, 4, 4, 128, 128, None) == 0
    cu = np.array([0, 3], np.int32)
    assert lib.fp_dense_attend_varlen(None, None, None, None, 0, 1, cu.ctypes.data, 4, 4, 128, 128, None) == -1
