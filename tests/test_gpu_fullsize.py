"""GPU parity at the full workload sizes (the launch configuration bench.py
times).  The GPU plans every head and attends every row; the oracle
recomputes a sample of heads one by one (bit-exact pattern, divergence,
line scores, estimate and block lists) and a sample of query-block rows of
attention (within the bf16 tolerance).  Every head's lists are checked for
the properties a plan has at any size."""
import numpy as np
import pytest

import oracle as O
from synth import BY_NAME, LayerGen
from tests._parity import check_attention, list_properties

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FULL = ["llama8b_32k", "llama8b_128k", "llama8b_128k_sparse", "glm9b_64k_bs64"]


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_long_context_last_amd as F
    return F


def sampled_heads(gen, want=("V", "QA", "N")):
    hs = []
    for t in want:
        if t in gen.types:
            hs.append(gen.types.index(t))
    return hs


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(F, name):
    cfg = BY_NAME[name]
    gen = LayerGen(cfg)
    print(f"[{name}] generating", flush=True)
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, q, k, v)
    outd = F.dense_attend(q, k, v, block=cfg.block) if name == "llama8b_32k" else None
    torch.cuda.synchronize()
    pattern, djs, row_ptr, col_idx = P.copy_out()
    info = P.info()
    colsum, diagsum, ahat, atrue = (P.debug(x) for x in ("colsum", "diagsum", "ahat", "atrue"))
    lists = P.lists()
    floor = O.floor_blocks(cfg.min_budget, cfg.block)
    for bh in range(cfg.B * cfg.Hq):
        list_properties(lists[bh], cfg.nb, floor)
    assert info.total_blocks == int(row_ptr[-1])
    print(f"[{name}] density {info.total_blocks / info.dense_blocks:.4f}, "
          f"query-aware heads {info.query_aware_heads}", flush=True)
    rng = np.random.default_rng(11)
    for h in sampled_heads(gen):
        kv = h // cfg.group
        qh, kh, vh = gen.q_head(0, h), gen.k_head(0, kv), gen.v_head(0, kv)
        hp = O.plan_head(qh, kh, cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
        print(f"[{name}] head {h} ({gen.types[h]}): D={hp.D:.5f} pattern={hp.pattern}", flush=True)
        np.testing.assert_array_equal(colsum[h], hp.stats.c)
        np.testing.assert_array_equal(diagsum[h], hp.stats.g)
        np.testing.assert_array_equal(atrue[h], hp.stats.a_true)
        np.testing.assert_array_equal(ahat[h], O.tri_values(hp.A))
        assert djs[h] == hp.D and int(pattern[h]) == hp.pattern
        for r in range(cfg.nb):
            assert np.array_equal(lists[h][r], hp.lists[r]), (h, r)
        rows = sorted(set([0, 1, cfg.nb // 2, cfg.nb - 1] + rng.choice(cfg.nb, 2, replace=False).tolist()))
        ref = O.attend_rows(qh, kh, vh, hp.mask, cfg.block, rows)
        refd = O.attend_rows(qh, kh, vh, O.dense_mask(cfg.nb), cfg.block, rows[:3]) if outd is not None else {}
        for r in rows:
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), ref[r], cfg.dtype, f"{name} h{h} row {r}")
            if r in refd:
                check_attention(outd[0, h, sl].float().cpu().numpy(), refd[r], cfg.dtype, f"dense h{h} row {r}")
    del q, k, v, out, outd, P
    torch.cuda.empty_cache()


EDGE = {
    # the largest supported row count, N / block = 4096 (block 64, N = 262144)
    "max_blocks_262k_bs64": BY_NAME["glm9b_64k_bs64"].with_(Hq=2, Hkv=1, N=262144, explicit_types=("V", "QA")),
    # just past the estimate kernel's 1024-block path (1025 blocks)
    "blocks_1025_bs64": BY_NAME["glm9b_64k_bs64"].with_(Hq=2, Hkv=1, N=1025 * 64, explicit_types=("QA", "N")),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_size_limits(F, name):
    cfg = EDGE[name]
    gen = LayerGen(cfg)
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, q, k, v)
    torch.cuda.synchronize()
    pattern, djs, _, _ = P.copy_out()
    colsum, diagsum, ahat, atrue = (P.debug(x) for x in ("colsum", "diagsum", "ahat", "atrue"))
    lists = P.lists()
    rng = np.random.default_rng(5)
    for h in range(cfg.Hq):
        hp = O.plan_head(gen.q_head(0, h), gen.k_head(0, 0), cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
        np.testing.assert_array_equal(colsum[h], hp.stats.c)
        np.testing.assert_array_equal(diagsum[h], hp.stats.g)
        np.testing.assert_array_equal(atrue[h], hp.stats.a_true)
        np.testing.assert_array_equal(ahat[h], O.tri_values(hp.A))
        assert djs[h] == hp.D and int(pattern[h]) == hp.pattern
        for r in range(cfg.nb):
            assert np.array_equal(lists[h][r], hp.lists[r]), (h, r)
        rows = sorted(set([0, cfg.nb - 1] + rng.choice(cfg.nb, 2, replace=False).tolist()))
        ref = O.attend_rows(gen.q_head(0, h), gen.k_head(0, 0), gen.v_head(0, 0), hp.mask, cfg.block, rows)
        for r in rows:
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), ref[r], cfg.dtype, f"{name} h{h} row {r}")


@pytest.mark.parametrize("name,max_budget,qa_selection", [("llama8b_32k", 4096, "flattened"),
                                                          ("glm9b_64k_bs64", 8192, "flattened"),
                                                          ("llama8b_128k", 0, "querywise"),
                                                          ("glm9b_64k_bs64", 0, "querywise")])
def test_full_size_plan_options(F, name, max_budget, qa_selection):
    """The optional settings at full size: every row within the cap, sampled
    heads' lists bit-exact with the oracle's plan under the same settings,
    sampled rows of attention."""
    cfg = BY_NAME[name]
    gen = LayerGen(cfg)
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
               max_budget=max_budget, qa_selection=qa_selection)
    out = F.attend(P, q, k, v)
    torch.cuda.synchronize()
    cap = O.cap_blocks(max_budget, cfg.block) or cfg.nb
    lists = P.lists()
    floor = O.floor_blocks(cfg.min_budget, cfg.block)
    for bh in range(cfg.B * cfg.Hq):
        list_properties(lists[bh], cfg.nb, floor)
        assert max(len(x) for x in lists[bh]) <= cap
    rng = np.random.default_rng(17)
    for h in sampled_heads(gen, ("V", "S", "QA")):
        kv = h // cfg.group
        qh, kh, vh = gen.q_head(0, h), gen.k_head(0, kv), gen.v_head(0, kv)
        hp = O.plan_head(qh, kh, cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, max_budget, qa_selection)
        print(f"[{name} cap {max_budget} {qa_selection}] head {h} ({gen.types[h]}): "
              f"{sum(len(x) for x in hp.lists)} blocks", flush=True)
        for r in range(cfg.nb):
            assert np.array_equal(lists[h][r], hp.lists[r]), (h, r)
        rows = sorted(set([cfg.nb - 1] + rng.choice(cfg.nb, 2, replace=False).tolist()))
        ref = O.attend_rows(qh, kh, vh, hp.mask, cfg.block, rows)
        for r in rows:
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), ref[r], cfg.dtype, f"{name} h{h} row {r}")
    del q, k, v, out, P
    torch.cuda.empty_cache()
