"""Plans exported to a file and replayed: a plan made on the GPU is written
with its intermediates (Plan.export), read back on the host
(plan_io.read), and the file alone is checked bit for bit against the CPU
oracle run on the same seeded inputs — as a plan saved in one session would
be checked in another."""
import numpy as np
import pytest

import oracle as O
from sparse_long_context_last_amd import plan_io
from synth import BY_NAME, LayerGen
from tests._parity import compare_head
from tests.test_gpu_ragged import packed
from tests.test_gpu_token import oracle_cols

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_long_context_last_amd as F
    return F


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16 if dtype == "bf16" else torch.float32)


def test_exported_plan_replays_against_the_oracle(F, tmp_path):
    cfg = BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=2048, mix=(0.25, 0.25, 0.25, 0.25))
    q, k, v = LayerGen(cfg).numpy_layer()
    P = F.plan(dev(q, cfg.dtype), dev(k, cfg.dtype), block=cfg.block, gamma=cfg.gamma, tau=cfg.tau,
               min_budget=cfg.min_budget)
    path = tmp_path / "plan.npz"
    P.export(path)
    P.destroy()
    f = plan_io.read(path)
    m = f["meta"]
    assert (m["Hq"], m["Hkv"], m["d"], m["block"], m["seqlens"], m["layout"], m["dtype"]) == \
        (cfg.Hq, cfg.Hkv, cfg.d, cfg.block, [cfg.N], "bhnd", "bf16")
    assert (m["gamma"], m["tau"], m["min_budget"]) == (cfg.gamma, cfg.tau, cfg.min_budget)
    dbg = {it: x[0] for it, x in f["intermediates"].items()}
    lists = plan_io.lists(f)
    group = cfg.Hq // cfg.Hkv
    for kv in range(cfg.Hkv):
        np.testing.assert_array_equal(dbg["kbar"][kv], O.pool_mean(k[0, kv], cfg.block))
    for h in range(cfg.Hq):
        hp = O.plan_head(q[0, h], k[0, h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
        compare_head(None, dbg, f["pattern"], f["djs"], lists, h, hp)
        np.testing.assert_array_equal(dbg["counts"][h], [len(x) for x in hp.lists])
    print(f"[export] {path.stat().st_size} bytes, {cfg.Hq} heads replayed", flush=True)


def test_exported_packed_token_plan(F, tmp_path):
    cfg = BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, explicit_types=("V", "V", "S", "QA"))
    lens = [700, 0, 1100, 64]
    seqs, (qc, kc, _), cu = packed(cfg, lens)
    P = F.plan_varlen(dev(qc, cfg.dtype), dev(kc, cfg.dtype), cu, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau,
                      min_budget=cfg.min_budget, vs_granularity="token")
    path = tmp_path / "packed.npz"
    P.export(path)
    f = plan_io.read(path)
    # the file holds exactly what the live plan reports
    for name, x in zip(("pattern", "djs", "row_ptr", "col_idx"), P.copy_out()):
        np.testing.assert_array_equal(f[name], x)
    for item in plan_io.ITEMS:
        for a, b in zip(f["intermediates"][item], P.debug_seqs(item)):
            assert (a is None and b is None) or np.array_equal(a, b), item
    assert f["meta"]["seqlens"] == lens and f["meta"]["vs_granularity"] == "token"
    assert f["meta"]["layout"] == "thd"
    # and replays against the oracle
    lists = plan_io.lists(f)
    for b, (q, k, _) in enumerate(seqs):
        if lens[b] == 0:
            assert all(len(lists[b * cfg.Hq + h]) == 0 for h in range(cfg.Hq))
            continue
        for h in range(cfg.Hq):
            bh = b * cfg.Hq + h
            hp = O.plan_head(q[h], k[0], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, vs_granularity="token")
            assert int(f["pattern"][bh]) == hp.pattern and f["djs"][bh] == hp.D
            for r in range(len(hp.lists)):
                assert np.array_equal(lists[bh][r], hp.lists[r]), (b, h, r)
            ptr, idx = oracle_cols(hp, cfg.block)
            np.testing.assert_array_equal(f["intermediates"]["colptr"][b][h], ptr)
            np.testing.assert_array_equal(f["intermediates"]["colidx"][b][h][: ptr[-1]], idx)
