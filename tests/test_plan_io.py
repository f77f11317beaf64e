"""The exported-plan file format (sparse_long_context_last_amd.plan_io) on the
host: a written plan reads back array for array, the per-row lists come out
as the CSR arrays say, and files that are not such a plan, are inconsistent
or would need unpickling are refused."""
import json

import numpy as np
import pytest

from sparse_long_context_last_amd import plan_io


def meta(**kw):
    m = dict(Hq=2, Hkv=1, d=64, block=64, seqlens=[130, 0, 64], layout="thd", dtype="bf16", gamma=0.9,
             tau=0.1, min_budget=128, max_budget=0, qa_selection="flattened", vs_granularity="block")
    m.update(kw)
    return m


def fake_plan(m, rng):
    bs, Hq = m["block"], m["Hq"]
    rows = [list(range(r + 1)) for L in m["seqlens"] for _ in range(Hq) for r in range(-(-L // bs))]
    row_ptr = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int32)
    col_idx = np.array([c for x in rows for c in x], np.int32)
    BH = len(m["seqlens"]) * Hq
    pattern = rng.integers(0, 2, BH).astype(np.uint8)
    djs = rng.random(BH)
    inter = {}
    for item, (shape, dt) in plan_io.ITEMS.items():
        if item in ("colptr", "colidx"):
            continue
        per = []
        for L in m["seqlens"]:
            nb = -(-L // bs)
            per.append(None if L == 0 else rng.random(shape(Hq, m["Hkv"], m["d"], bs, L, nb)).astype(dt))
        inter[item] = per
    return pattern, djs, row_ptr, col_idx, inter, rows


def test_round_trip(tmp_path):
    rng = np.random.default_rng(3)
    m = meta()
    pattern, djs, row_ptr, col_idx, inter, rows = fake_plan(m, rng)
    f = tmp_path / "p.npz"
    plan_io.write(f, m, pattern, djs, row_ptr, col_idx, inter)
    back = plan_io.read(f)
    assert back["meta"] == m
    for name, x in (("pattern", pattern), ("djs", djs), ("row_ptr", row_ptr), ("col_idx", col_idx)):
        np.testing.assert_array_equal(back[name], x)
        assert back[name].dtype == x.dtype
    for item, per in inter.items():
        for a, b in zip(back["intermediates"][item], per):
            assert (a is None and b is None) or np.array_equal(a, b)
    got = plan_io.lists(back)
    assert [list(r) for h in got for r in h] == rows


def test_plan_without_intermediates(tmp_path):
    rng = np.random.default_rng(4)
    m = meta(seqlens=[200], layout="bhnd")
    pattern, djs, row_ptr, col_idx, _, _ = fake_plan(m, rng)
    plan_io.write(tmp_path / "p.npz", m, pattern, djs, row_ptr, col_idx)
    assert plan_io.read(tmp_path / "p.npz")["intermediates"] == {}


def test_inconsistent_plans_are_refused(tmp_path):
    rng = np.random.default_rng(5)
    m = meta()
    pattern, djs, row_ptr, col_idx, inter, _ = fake_plan(m, rng)
    with pytest.raises(plan_io.PlanFileError):
        plan_io.write(tmp_path / "a.npz", m, pattern[:-1], djs, row_ptr, col_idx)
    with pytest.raises(plan_io.PlanFileError):
        plan_io.write(tmp_path / "b.npz", m, pattern, djs, row_ptr, col_idx[:-1])
    bad = dict(inter)
    bad["qbar"] = [x[:, :1] if x is not None else None for x in inter["qbar"]]
    with pytest.raises(plan_io.PlanFileError):
        plan_io.write(tmp_path / "c.npz", m, pattern, djs, row_ptr, col_idx, bad)
    with pytest.raises(plan_io.PlanFileError):
        plan_io.write(tmp_path / "d.npz", {k: v for k, v in m.items() if k != "gamma"}, pattern, djs, row_ptr,
                      col_idx)


def test_foreign_files_are_refused(tmp_path):
    np.savez(tmp_path / "other.npz", x=np.zeros(3))
    with pytest.raises(plan_io.PlanFileError):
        plan_io.read(tmp_path / "other.npz")
    # a file carrying a pickled object array is not unpickled
    np.savez(tmp_path / "obj.npz", format=np.array(plan_io.FORMAT), meta=np.array(json.dumps(meta())),
             pattern=np.array([object()], dtype=object))
    with pytest.raises(ValueError):
        plan_io.read(tmp_path / "obj.npz")
