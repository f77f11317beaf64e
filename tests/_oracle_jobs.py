"""Oracle work for the full-size GPU parity tests, run in worker processes.

Every job regenerates one query head (and its key/value head) from the
seeded generator and runs the CPU oracle on it, so the workers need nothing
from the GPU process and can run while the GPU plans the layer.  Workers are
started with the "spawn" method (a fresh interpreter that never touches the
GPU) and limit their BLAS threads to one each.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:   # pragma: no cover - threadpoolctl is optional
        pass


def make_pool(max_workers: int | None = None) -> ProcessPoolExecutor:
    """A pool sized to the CPUs this process may use (at most 16)."""
    n = max_workers or max(1, min(16, len(os.sched_getaffinity(0))))
    return ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_init_worker)


def oracle_head(cfg, h: int, rows, plan_kw: dict | None = None, dense_rows=(), L: int | None = None,
                b: int = 0) -> dict:
    """The oracle's plan of query head h of sequence b of layer ``cfg`` and its
    float64 attention on the query-block rows ``rows`` (and dense causal
    attention on ``dense_rows``); with ``L`` the head's first L tokens only
    (a sequence of a packed batch).  Lists come back flattened with per-row
    counts."""
    import oracle as O
    from synth import LayerGen

    gen = LayerGen(cfg)
    kv = h // cfg.group
    qh, kh, vh = gen.q_head(b, h), gen.k_head(b, kv), gen.v_head(b, kv)
    if L is not None:
        qh, kh, vh = qh[:L], kh[:L], vh[:L]
    hp = O.plan_head(qh, kh, cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, **(plan_kw or {}))
    ref = O.attend_rows(qh, kh, vh, hp.mask, cfg.block, list(rows), hp.cols) if len(rows) else {}
    refd = O.attend_rows(qh, kh, vh, O.dense_mask(cfg.nb), cfg.block, list(dense_rows)) if len(dense_rows) else {}
    counts = np.array([len(x) for x in hp.lists], dtype=np.int64)
    flat = np.concatenate(hp.lists).astype(np.int32) if len(hp.lists) else np.zeros(0, np.int32)
    return dict(h=h, type=gen.types[h], pattern=hp.pattern, D=hp.D, qbar=hp.qbar, kbar=hp.kbar,
                M=hp.stats.M, Z=hp.stats.Z, c=hp.stats.c, g=hp.stats.g, a_true=hp.stats.a_true,
                ahat=O.tri_values(hp.A), counts=counts, flat=flat, ref=ref, refd=refd,
                blocks=int(counts.sum()),
                cols=(np.nonzero(hp.cols)[0].astype(np.int32) if hp.cols is not None else np.zeros(0, np.int32)))
