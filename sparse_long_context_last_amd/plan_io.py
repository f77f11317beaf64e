"""Plans on disk: a plan's host copy written to one ``.npz`` file and read back.

An exported plan holds what fp_plan_copy_out returns (pattern, divergence D,
CSR block lists) and, optionally, every intermediate of pattern
determination and selection (fp_plan_copy_debug), together with the shapes
and hyper-parameters it was made with.  Such a file lets a plan made on the
GPU be checked again later, on any host, against an independent
implementation of the method run on the same inputs (a replay), or compared
with a plan made by another build.

Only plain arrays are stored (numeric arrays and one JSON string), so the
file is read with ``numpy.load(allow_pickle=False)``; nothing in it is
executed.  This module uses numpy alone: it needs no GPU.
"""
from __future__ import annotations

import json
from typing import Dict, List, Optional

import numpy as np

FORMAT = "flexprefill-plan/1"

# intermediates per sequence: item -> (shape from (Hq, Hkv, d, block, L, nb), dtype)
ITEMS = {
    "qbar": (lambda Hq, Hkv, d, bs, L, nb: (Hq, nb, d), np.float32),
    "kbar": (lambda Hq, Hkv, d, bs, L, nb: (Hkv, nb, d), np.float32),
    "rowmax": (lambda Hq, Hkv, d, bs, L, nb: (Hq, bs), np.float32),
    "rowsum": (lambda Hq, Hkv, d, bs, L, nb: (Hq, bs), np.float32),
    "colsum": (lambda Hq, Hkv, d, bs, L, nb: (Hq, L), np.float32),
    "diagsum": (lambda Hq, Hkv, d, bs, L, nb: (Hq, L), np.float32),
    "atrue": (lambda Hq, Hkv, d, bs, L, nb: (Hq, nb), np.float32),
    "ahat": (lambda Hq, Hkv, d, bs, L, nb: (Hq, nb * (nb + 1) // 2), np.float32),
    "counts": (lambda Hq, Hkv, d, bs, L, nb: (Hq, nb), np.int32),
    # token-granular vertical lines only
    "colptr": (lambda Hq, Hkv, d, bs, L, nb: (Hq, nb + 1), np.int32),
    "colidx": (lambda Hq, Hkv, d, bs, L, nb: (Hq, L), np.int32),
}

_META_KEYS = ("Hq", "Hkv", "d", "block", "seqlens", "layout", "dtype", "gamma", "tau", "min_budget",
              "max_budget", "qa_selection", "vs_granularity")


class PlanFileError(ValueError):
    """The file is not an exported plan of this format, or is inconsistent."""


def _rows(meta: dict) -> int:
    bs = meta["block"]
    return sum(-(-L // bs) for L in meta["seqlens"]) * meta["Hq"]


def write(path, meta: dict, pattern: np.ndarray, djs: np.ndarray, row_ptr: np.ndarray,
          col_idx: np.ndarray, intermediates: Optional[Dict[str, List[Optional[np.ndarray]]]] = None) -> None:
    """Write one plan.  `meta` holds the keys of _META_KEYS; `intermediates`
    maps an item of ITEMS to a list over sequences of arrays (None for an
    empty sequence)."""
    missing = [k for k in _META_KEYS if k not in meta]
    if missing:
        raise PlanFileError(f"meta lacks {missing}")
    m = {k: meta[k] for k in _META_KEYS}
    m["seqlens"] = [int(x) for x in m["seqlens"]]
    arrays = {
        "format": np.array(FORMAT),
        "meta": np.array(json.dumps(m, sort_keys=True)),
        "pattern": np.ascontiguousarray(pattern, np.uint8),
        "djs": np.ascontiguousarray(djs, np.float64),
        "row_ptr": np.ascontiguousarray(row_ptr, np.int32),
        "col_idx": np.ascontiguousarray(col_idx, np.int32),
    }
    for item, per_seq in (intermediates or {}).items():
        if item not in ITEMS:
            raise PlanFileError(f"unknown intermediate {item!r}")
        for b, x in enumerate(per_seq):
            if x is not None:
                arrays[f"{item}.{b}"] = np.ascontiguousarray(x, ITEMS[item][1])
    _validate(m, arrays)
    with open(path, "wb") as f:
        np.savez(f, **arrays)


def read(path) -> dict:
    """Read a plan written by write(): a dict with 'meta' (dict), 'pattern',
    'djs', 'row_ptr', 'col_idx' and 'intermediates' ({item: [per sequence
    array or None]})."""
    with np.load(path, allow_pickle=False) as z:
        arrays = {k: z[k] for k in z.files}
    if "format" not in arrays or str(arrays["format"]) != FORMAT:
        raise PlanFileError(f"not a {FORMAT} file")
    try:
        meta = json.loads(str(arrays["meta"]))
    except (KeyError, json.JSONDecodeError) as e:
        raise PlanFileError(f"bad meta record: {e}") from None
    _validate(meta, arrays)
    inter: Dict[str, List[Optional[np.ndarray]]] = {}
    for item in ITEMS:
        per = [arrays.get(f"{item}.{b}") for b in range(len(meta["seqlens"]))]
        if any(x is not None for x in per):
            inter[item] = per
    return {"meta": meta, "pattern": arrays["pattern"], "djs": arrays["djs"], "row_ptr": arrays["row_ptr"],
            "col_idx": arrays["col_idx"], "intermediates": inter}


def _validate(meta: dict, arrays: dict) -> None:
    for k in _META_KEYS:
        if k not in meta:
            raise PlanFileError(f"meta lacks {k!r}")
    Hq, Hkv, d, bs = (int(meta[k]) for k in ("Hq", "Hkv", "d", "block"))
    seqlens = [int(x) for x in meta["seqlens"]]
    BH = len(seqlens) * Hq
    if arrays["pattern"].shape != (BH,) or arrays["djs"].shape != (BH,):
        raise PlanFileError("pattern and djs must hold one entry per (sequence, query head)")
    rows = _rows(meta)
    rp, ci = arrays["row_ptr"], arrays["col_idx"]
    if rp.shape != (rows + 1,) or rp[0] != 0 or np.any(np.diff(rp) < 0) or rp[-1] != ci.size:
        raise PlanFileError("row_ptr is not a CSR offset array over the plan's rows")
    for key, x in arrays.items():
        if "." not in key:
            continue
        item, b = key.split(".", 1)
        if item not in ITEMS or not b.isdigit() or int(b) >= len(seqlens):
            raise PlanFileError(f"unexpected array {key!r}")
        L = seqlens[int(b)]
        want = ITEMS[item][0](Hq, Hkv, d, bs, L, -(-L // bs))
        if x.shape != want or x.dtype != ITEMS[item][1]:
            raise PlanFileError(f"{key}: shape {x.shape} {x.dtype}, expected {want} {np.dtype(ITEMS[item][1])}")


def lists(plan_file: dict) -> List[List[np.ndarray]]:
    """Per (sequence b, head h), index b * Hq + h: the per-row arrays of
    selected key blocks (ascending), as Plan.lists() returns them."""
    meta, rp, ci = plan_file["meta"], plan_file["row_ptr"], plan_file["col_idx"]
    bs, Hq = meta["block"], meta["Hq"]
    out, i = [], 0
    for L in meta["seqlens"]:
        nb = -(-L // bs)
        for _ in range(Hq):
            rows = []
            for _ in range(nb):
                rows.append(ci[rp[i]: rp[i + 1]].copy())
                i += 1
            out.append(rows)
    return out
