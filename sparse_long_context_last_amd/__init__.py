"""FlexPrefill sparse pre-filling attention for one layer on an MI355X (gfx950).

Thin Python binding over the C ABI of ``libfp_prefill.so`` (include/fp_prefill.h):
torch tensors only provide device memory and the current HIP stream; every
step of the method runs in the library's HIP kernels.

    plan = plan(q, k, block=128, gamma=0.95, tau=0.1, min_budget=1024)
    o = attend(plan, q, k, v)          # block-sparse causal attention
    o_dense = dense_attend(q, k, v, block=128)
    # packed sequences of different lengths: q [T, Hq, d], k, v [T, Hkv, d]
    p = plan_varlen(q, k, cu_seqlens, block=128)
    o = attend(p, q, k, v)
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np

from . import _lib
from ._lib import FpError, PlanInfo  # noqa: F401

__all__ = ["Plan", "plan", "plan_varlen", "attend", "dense_attend", "dense_attend_varlen",
           "profile_enable", "profile_read", "canonical_constants", "workspace_trim", "FpError"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.FP_BF16
    if t.dtype == torch.float32:
        return _lib.FP_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(t, name: str, ndim: int = 4) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be " + ("[B, H, N, d]" if ndim == 4 else "[T, H, d]"))


def _stream_ptr(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _cu_array(cu_seqlens) -> np.ndarray:
    """Host int32 copy of cu_seqlens (list, numpy array or CPU tensor)."""
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-d array of nseq + 1 offsets")
    if cu.max(initial=0) > np.iinfo(np.int32).max:
        raise ValueError("cu_seqlens exceeds int32")
    return cu.astype(np.int32)


class Plan:
    """Device-resident FlexPrefill plan (pattern per head, block lists)."""

    def __init__(self, handle: C.c_void_p, Hq, Hkv, d, block, seqlens, layout: int, dtype_code: int, stream,
                 N: Optional[int] = None, params: Optional[dict] = None):
        self._h = handle
        self.params = dict(params or {})      # gamma, tau, min_budget, max_budget, qa_selection, vs_granularity
        self.Hq, self.Hkv, self.d, self.block = Hq, Hkv, d, block
        self.seqlens = [int(x) for x in seqlens]
        self.layout = layout
        self.B = len(self.seqlens)
        self.N = max(self.seqlens, default=0) if N is None else int(N)
        self.nb = -(-self.N // block) if block else 0
        self.nbs = [-(-L // block) for L in self.seqlens]
        self.dtype_code = dtype_code
        self._stream = stream

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("plan has been destroyed")
        return self._h

    def info(self) -> PlanInfo:
        out = PlanInfo()
        _lib.check(_lib.load().fp_plan_info_get(self.handle, C.byref(out)), "fp_plan_info_get")
        return out

    def copy_out(self):
        """(pattern [B*Hq] uint8, djs [B*Hq] float64, row_ptr, col_idx) on the host."""
        inf = self.info()
        BH = self.B * self.Hq
        pattern = np.zeros(BH, np.uint8)
        djs = np.zeros(BH, np.float64)
        row_ptr = np.zeros(inf.rows + 1, np.int32)
        col_idx = np.zeros(max(inf.total_blocks, 1), np.int32)
        _lib.check(_lib.load().fp_plan_copy_out(
            self.handle, pattern.ctypes.data, djs.ctypes.data, row_ptr.ctypes.data,
            col_idx.ctypes.data, _stream_ptr(self._stream)), "fp_plan_copy_out")
        return pattern, djs, row_ptr, col_idx[: inf.total_blocks]

    def lists(self):
        """Per (b*Hq + h) a list of per-row int32 arrays of key-block indices
        (sequence b has ceil(L_b / block) rows)."""
        pattern, djs, row_ptr, col_idx = self.copy_out()
        out = []
        i = 0
        for b in range(self.B):
            for h in range(self.Hq):
                rows = []
                for r in range(self.nbs[b]):
                    rows.append(col_idx[row_ptr[i]: row_ptr[i + 1]].copy())
                    i += 1
                out.append(rows)
        return out

    def _item_shape(self, item: str, L: int, nb: int):
        d, bs = self.d, self.block
        return {"qbar": ((self.Hq, nb, d), np.float32), "kbar": ((self.Hkv, nb, d), np.float32),
                "rowmax": ((self.Hq, bs), np.float32), "rowsum": ((self.Hq, bs), np.float32),
                "colsum": ((self.Hq, L), np.float32), "diagsum": ((self.Hq, L), np.float32),
                "atrue": ((self.Hq, nb), np.float32), "ahat": ((self.Hq, nb * (nb + 1) // 2), np.float32),
                "counts": ((self.Hq, nb), np.int32),
                "colptr": ((self.Hq, nb + 1), np.int32), "colidx": ((self.Hq, L), np.int32)}[item]

    def debug_seqs(self, item: str):
        """An intermediate of steps 1-2 per sequence: a list over sequences of
        arrays [Hq, ...] ([Hkv, ...] for kbar), None for an empty sequence."""
        parts, total, dt = [], 0, np.float32
        for L, nb in zip(self.seqlens, self.nbs):
            shape, dt = self._item_shape(item, L, nb)
            parts.append(shape if L > 0 else None)
            total += int(np.prod(shape)) if L > 0 else 0
        flat = np.zeros(total, dt)
        _lib.check(_lib.load().fp_plan_copy_debug(self.handle, _lib.DEBUG_ITEMS[item],
                                                  flat.ctypes.data, flat.nbytes), "fp_plan_copy_debug")
        out, o = [], 0
        for shape in parts:
            if shape is None:
                out.append(None)
                continue
            n = int(np.prod(shape))
            out.append(flat[o: o + n].reshape(shape))
            o += n
        return out

    def debug(self, item: str) -> np.ndarray:
        """An intermediate for sequences of one length, stacked over
        (b, head): [B*Hq, ...] ([B*Hkv, ...] for kbar)."""
        if len(set(self.seqlens)) > 1:
            raise ValueError("sequences differ in length: use debug_seqs")
        parts = [x for x in self.debug_seqs(item) if x is not None]
        if not parts:
            shape, dt = self._item_shape(item, self.N, self.nb)
            return np.zeros((0,) + shape[1:], dt)
        return np.concatenate(parts, axis=0)

    def export(self, path, intermediates: bool = True) -> None:
        """Write the plan's host copy to an .npz file (plan_io format): the
        pattern, D and block lists of every head, the shapes and parameters
        it was made with and, with `intermediates`, every selection
        intermediate, so that it can be replayed against another
        implementation later (plan_io.read)."""
        from . import plan_io
        pattern, djs, row_ptr, col_idx = self.copy_out()
        meta = dict(Hq=self.Hq, Hkv=self.Hkv, d=self.d, block=self.block, seqlens=self.seqlens,
                    layout="bhnd" if self.layout == _lib.FP_LAYOUT_BHND else "thd",
                    dtype="bf16" if self.dtype_code == _lib.FP_BF16 else "fp32", **self.params)
        inter = None
        if intermediates:
            items = [it for it in plan_io.ITEMS
                     if it not in ("colptr", "colidx") or self.params.get("vs_granularity") == "token"]
            inter = {it: self.debug_seqs(it) for it in items}
        plan_io.write(path, meta, pattern, djs, row_ptr, col_idx, inter)

    def destroy(self) -> None:
        if self._h is not None:
            _lib.load().fp_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _options(max_budget: int, qa_selection: str, vs_granularity: str):
    if qa_selection not in _lib.QA_SELECTION:
        raise ValueError(f"qa_selection must be one of {sorted(_lib.QA_SELECTION)}")
    if vs_granularity not in _lib.VS_GRANULARITY:
        raise ValueError(f"vs_granularity must be one of {sorted(_lib.VS_GRANULARITY)}")
    return _lib.PlanOptions(int(max_budget), _lib.QA_SELECTION[qa_selection],
                            _lib.VS_GRANULARITY[vs_granularity])


def _params(gamma, tau, min_budget, max_budget, qa_selection, vs_granularity) -> dict:
    return dict(gamma=float(gamma), tau=float(tau), min_budget=int(min_budget), max_budget=int(max_budget),
                qa_selection=str(qa_selection), vs_granularity=str(vs_granularity))


def plan(q, k, block: int = 128, gamma: float = 0.95, tau: float = 0.1,
         min_budget: int = 1024, max_budget: int = 0, qa_selection: str = "flattened",
         vs_granularity: str = "block", stream=None) -> Plan:
    """Pattern determination and index selection for q [B, Hq, N, d],
    k [B, Hkv, N, d] (fp_prefill_plan_ex; max_budget = 0 leaves rows
    uncapped; qa_selection "flattened" or "querywise"; vs_granularity
    "block" or "token")."""
    _check_tensor(q, "q")
    _check_tensor(k, "k")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d):
        raise ValueError("k must be [B, Hkv, N, d] with q's B, N and d")
    dt = _dtype_code(q)
    opts = _options(max_budget, qa_selection, vs_granularity)
    h = C.c_void_p()
    _lib.check(_lib.load().fp_prefill_plan_ex(q.data_ptr(), k.data_ptr(), dt, B, Hq, Hkv, N, d, block,
                                              float(gamma), float(tau), int(min_budget), C.byref(opts),
                                              _stream_ptr(stream), C.byref(h)), "fp_prefill_plan_ex")
    return Plan(h, Hq, Hkv, d, block, [N] * B, _lib.FP_LAYOUT_BHND, dt, stream, N=N,
                params=_params(gamma, tau, min_budget, max_budget, qa_selection, vs_granularity))


def plan_varlen(q, k, cu_seqlens, block: int = 128, gamma: float = 0.95, tau: float = 0.1,
                min_budget: int = 1024, max_budget: int = 0, qa_selection: str = "flattened",
                vs_granularity: str = "block", stream=None) -> Plan:
    """The same for packed sequences: q [T, Hq, d], k [T, Hkv, d], sequence b
    at tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 (fp_prefill_plan_varlen)."""
    _check_tensor(q, "q", 3)
    _check_tensor(k, "k", 3)
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    cu = _cu_array(cu_seqlens)
    if tuple(k.shape) != (T, Hkv, d) or int(cu[-1]) != T:
        raise ValueError("k must be [T, Hkv, d] and cu_seqlens[-1] must equal T")
    dt = _dtype_code(q)
    opts = _options(max_budget, qa_selection, vs_granularity)
    h = C.c_void_p()
    _lib.check(_lib.load().fp_prefill_plan_varlen(q.data_ptr(), k.data_ptr(), dt, cu.size - 1, cu.ctypes.data,
                                                  Hq, Hkv, d, block, float(gamma), float(tau), int(min_budget),
                                                  C.byref(opts), _stream_ptr(stream), C.byref(h)),
               "fp_prefill_plan_varlen")
    return Plan(h, Hq, Hkv, d, block, np.diff(cu).tolist(), _lib.FP_LAYOUT_THD, dt, stream,
                params=_params(gamma, tau, min_budget, max_budget, qa_selection, vs_granularity))


def attend(p: Plan, q, k, v, out=None, stream=None, noalloc: bool = False):
    """Block-sparse causal attention over the plan's selection (fp_prefill_attend;
    with noalloc, fp_prefill_attend_noalloc: no device allocation, the
    library's static workspace of 64 MiB per GPU).  ``out`` must be given
    for a call that may not allocate."""
    torch = _torch()
    ndim = 4 if p.layout == _lib.FP_LAYOUT_BHND else 3
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, ndim)
    if ndim == 4:
        ok = tuple(q.shape) == (p.B, p.Hq, p.N, p.d) and tuple(k.shape) == (p.B, p.Hkv, p.N, p.d)
    else:
        T = sum(p.seqlens)
        ok = tuple(q.shape) == (T, p.Hq, p.d) and tuple(k.shape) == (T, p.Hkv, p.d)
    if not ok or k.shape != v.shape:
        raise ValueError("q / k / v shapes do not match the plan")
    if _dtype_code(q) != p.dtype_code or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must have the plan's dtype")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", ndim)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q")
    name = "fp_prefill_attend_noalloc" if noalloc else "fp_prefill_attend"
    _lib.check(getattr(_lib.load(), name)(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), _stream_ptr(stream)), name)
    return out


def dense_attend(q, k, v, block: int = 128, out=None, stream=None):
    """Full causal attention with the same tile kernel (fp_dense_attend)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or k.shape != v.shape:
        raise ValueError("k and v must be [B, Hkv, N, d]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _lib.check(_lib.load().fp_dense_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           dt, B, Hq, Hkv, N, d, block, _stream_ptr(stream)),
               "fp_dense_attend")
    return out


def dense_attend_varlen(q, k, v, cu_seqlens, block: int = 128, out=None, stream=None):
    """Full causal attention of packed sequences (fp_dense_attend_varlen)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, 3)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    cu = _cu_array(cu_seqlens)
    if tuple(k.shape) != (T, Hkv, d) or k.shape != v.shape or int(cu[-1]) != T:
        raise ValueError("k and v must be [T, Hkv, d] and cu_seqlens[-1] must equal T")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _lib.check(_lib.load().fp_dense_attend_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                  dt, cu.size - 1, cu.ctypes.data, Hq, Hkv, d, block,
                                                  _stream_ptr(stream)), "fp_dense_attend_varlen")
    return out


def workspace_trim() -> None:
    """Free the device memory the library keeps cached for reuse (see
    fp_workspace_trim); live plans keep their buffers."""
    _lib.check(_lib.load().fp_workspace_trim(), "fp_workspace_trim")


def profile_enable(on: bool = True) -> None:
    _lib.check(_lib.load().fp_profile_enable(1 if on else 0), "fp_profile_enable")


def profile_read(reset: bool = True):
    """(sparse_ms, sparse_launches, dense_ms, dense_launches): the attention
    kernel's summed time in ms and its number of launches since the last
    reset (divide for the average launch)."""
    sm, dm = C.c_double(), C.c_double()
    sn, dn = C.c_longlong(), C.c_longlong()
    _lib.check(_lib.load().fp_profile_read(C.byref(sm), C.byref(sn), C.byref(dm), C.byref(dn),
                                           1 if reset else 0), "fp_profile_read")
    return sm.value, sn.value, dm.value, dn.value


def canonical_constants(d: int = 128) -> dict:
    e2 = np.zeros(8, np.float32)
    lnc = np.zeros(11, np.float64)
    ln2, sh = C.c_double(), C.c_double()
    cs = C.c_float()
    _lib.check(_lib.load().fp_canonical_constants(d, e2.ctypes.data, lnc.ctypes.data, C.byref(ln2),
                                                  C.byref(sh), C.byref(cs)), "fp_canonical_constants")
    return {"e2": e2, "lnc": lnc, "ln2": ln2.value, "sqrt_half": sh.value,
            "C": np.float32(cs.value)}
