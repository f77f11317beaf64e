"""GPU parity at the full workload sizes (the launch configuration bench.py
times).  The GPU plans every head and attends every row.  The oracle
recomputes EVERY head of the four large layers, one head per worker process
(pattern, divergence, pooled vectors, last-block statistics, line scores,
true and estimated distributions and every row's block list, all bit-exact),
and at least two query-block rows of attention per head (within the bf16
tolerance); the planted-type representatives get more rows.  Every head's
lists are also checked for the properties a plan has at any size."""
import numpy as np
import pytest

import oracle as O
from synth import BY_NAME, LayerGen
from tests._oracle_jobs import make_pool, oracle_head
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


@pytest.fixture(scope="module")
def pool():
    ex = make_pool()
    yield ex
    ex.shutdown(wait=True, cancel_futures=True)


def representatives(gen):
    """The first head of each planted type."""
    return {gen.types.index(t) for t in ("V", "S", "QA", "N") if t in gen.types}


def row_sample(cfg, h, many: bool):
    """Query-block rows of head h whose attention the oracle recomputes: the
    last (longest) row and one seeded random row; more for representatives."""
    rng = np.random.default_rng([31, h])
    rows = {cfg.nb - 1, int(rng.integers(0, cfg.nb))}
    if many:
        rows |= {0, 1, cfg.nb // 2}
    return sorted(rows)


def compare_full_head(name, ref, gpu, bh):
    """Bit-exact comparison of one head's plan with the oracle's."""
    h = ref["h"]
    where = f"{name} head {h} ({ref['type']})"
    assert int(gpu["pattern"][bh]) == ref["pattern"], where
    assert gpu["djs"][bh] == ref["D"], (where, gpu["djs"][bh], ref["D"])
    np.testing.assert_array_equal(gpu["qbar"][bh], ref["qbar"], err_msg=where)
    np.testing.assert_array_equal(gpu["kbar"][gpu["kvof"](bh)], ref["kbar"], err_msg=where)
    np.testing.assert_array_equal(gpu["rowmax"][bh], ref["M"], err_msg=where)
    np.testing.assert_array_equal(gpu["rowsum"][bh], ref["Z"], err_msg=where)
    np.testing.assert_array_equal(gpu["colsum"][bh], ref["c"], err_msg=where)
    np.testing.assert_array_equal(gpu["diagsum"][bh], ref["g"], err_msg=where)
    np.testing.assert_array_equal(gpu["atrue"][bh], ref["a_true"], err_msg=where)
    np.testing.assert_array_equal(gpu["ahat"][bh], ref["ahat"], err_msg=where)
    rp = gpu["row_ptr"]
    nb = len(ref["counts"])
    got_counts = np.diff(rp[bh * nb: (bh + 1) * nb + 1])
    np.testing.assert_array_equal(got_counts, ref["counts"], err_msg=where + ": row counts")
    np.testing.assert_array_equal(gpu["col_idx"][rp[bh * nb]: rp[(bh + 1) * nb]], ref["flat"],
                                  err_msg=where + ": block lists")


def gpu_plan_arrays(P, cfg):
    pattern, djs, row_ptr, col_idx = P.copy_out()
    out = dict(pattern=pattern, djs=djs, row_ptr=row_ptr, col_idx=col_idx,
               kvof=lambda bh: (bh // cfg.Hq) * cfg.Hkv + (bh % cfg.Hq) // cfg.group)
    for x in ("qbar", "kbar", "rowmax", "rowsum", "colsum", "diagsum", "atrue", "ahat"):
        out[x] = P.debug(x)
    return out


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(F, pool, name):
    run_layer(F, pool, name, BY_NAME[name])


# Head dimension 64 at sizes well past the small parity layers: every head
# bit-exact, as above (block 128 with GQA 4:1; block 64 with 16 query heads
# per key/value head).
D64 = {
    "llama8b_d64_16k": BY_NAME["llama8b_32k"].with_(N=16384, d=64),
    "glm9b_d64_16k_bs64": BY_NAME["glm9b_64k_bs64"].with_(N=16384, d=64, min_budget=1024),
}


@pytest.mark.parametrize("name", list(D64))
def test_full_head_parity_d64(F, pool, name):
    run_layer(F, pool, name, D64[name])


# fp32 inputs (vector-ALU last-block scores, fp32-MFMA attention) well past the
# small layers: a 16k layer with GQA 4:1 at block 128 and a 16k layer at block
# 64, every head bit-exact as above, sampled rows within 1e-4.
FP32 = {
    "fp32_gqa_16k": BY_NAME["tiny_fp32_4k"].with_(N=16384, Hq=8, Hkv=2, explicit_types=("V", "S", "QA", "N") * 2),
    "fp32_bs64_16k": BY_NAME["tiny_fp32_4k"].with_(N=16384, block=64, min_budget=512),
}


@pytest.mark.parametrize("name", list(FP32))
def test_full_head_parity_fp32(F, pool, name):
    run_layer(F, pool, name, FP32[name])


def test_full_size_two_sequences(F, pool):
    """The batched [B, H, N, d] layout with two sequences in one plan at 16k:
    every head of both sequences bit-exact, sampled rows within tolerance."""
    cfg = BY_NAME["llama8b_32k"].with_(B=2, N=16384, Hq=8, Hkv=2, mix=(0.25, 0.25, 0.25, 0.25))
    jobs = {}
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            rng = np.random.default_rng([41, b, h])
            rows = sorted({cfg.nb - 1, int(rng.integers(0, cfg.nb))})
            jobs[b, h] = pool.submit(oracle_head, cfg, h, rows, None, (), None, b)
    q, k, v = LayerGen(cfg).torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, q, k, v)
    torch.cuda.synchronize()
    gpu = gpu_plan_arrays(P, cfg)
    for (b, h), fut in jobs.items():
        ref = fut.result()
        compare_full_head(f"two sequences: seq {b}", ref, gpu, b * cfg.Hq + h)
        for r, want in ref["ref"].items():
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[b, h, sl].float().cpu().numpy(), want, cfg.dtype, f"seq {b} h{h} row {r}")
    print(f"[two sequences] {len(jobs)} heads bit-exact", flush=True)


# A packed batch of sequences of different lengths (ragged tails, an empty
# sequence) at sizes well past the small ragged layers: every head of every
# sequence bit-exact, sampled rows within tolerance.
PACKED = {
    "gqa_6seq": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, mix=(0.25, 0.25, 0.25, 0.25)),
                 [16384, 5003, 0, 777, 9000, 200]),
    # the packed batch bench.py --varlen times (128713 tokens, 32 query heads)
    "bench_varlen_7seq": (BY_NAME["llama8b_128k"], [65536, 33000, 16500, 8300, 4200, 1100, 77]),
}


@pytest.mark.parametrize("name", list(PACKED))
def test_full_size_packed_batch(F, pool, name):
    from tests.test_gpu_ragged import packed
    cfg, lens = PACKED[name]
    gens = [cfg.with_(B=1, N=max(128, -(-max(L, 1) // 128) * 128), seed=cfg.seed + 7 * b) for b, L in enumerate(lens)]
    jobs = {}
    for b, L in enumerate(lens):
        if L == 0:
            continue
        nbL = -(-L // cfg.block)
        for h in range(cfg.Hq):
            rng = np.random.default_rng([37, b, h])
            rows = sorted({nbL - 1, int(rng.integers(0, nbL))})
            jobs[b, h] = pool.submit(oracle_head, gens[b], h, rows, None, (), L)
    seqs, (qc, kc, vc), cu = packed(cfg, lens)
    dt = torch.bfloat16
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (qc, kc, vc))
    P = F.plan_varlen(qd, kd, cu, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, qd, kd, vd).float().cpu().numpy()
    pattern, djs, row_ptr, col_idx = P.copy_out()
    dbg = {x: P.debug_seqs(x) for x in ("qbar", "kbar", "rowmax", "rowsum", "colsum", "diagsum", "atrue", "ahat")}
    r0 = 0
    nchecked = 0
    for b, L in enumerate(lens):
        nbL = -(-L // cfg.block)
        rows_b = cfg.Hq * nbL
        if L == 0:
            assert not pattern[b * cfg.Hq:(b + 1) * cfg.Hq].any()
            continue
        rp = row_ptr[r0: r0 + rows_b + 1] - row_ptr[r0]
        ci = col_idx[row_ptr[r0]: row_ptr[r0 + rows_b]]
        seq_dbg = {x: dbg[x][b] for x in dbg}
        if L < cfg.block:
            # the plan keeps `block` representative rows; the first ones do not exist and hold 0
            for x in ("rowmax", "rowsum"):
                assert not seq_dbg[x][:, : cfg.block - L].any()
                seq_dbg[x] = seq_dbg[x][:, cfg.block - L:]
        gpu = dict(pattern=pattern[b * cfg.Hq:(b + 1) * cfg.Hq], djs=djs[b * cfg.Hq:(b + 1) * cfg.Hq],
                   row_ptr=rp, col_idx=ci, kvof=lambda h: h // cfg.group, **seq_dbg)
        for h in range(cfg.Hq):
            ref = jobs[b, h].result()
            compare_full_head(f"{name} seq {b} (L={L})", ref, gpu, h)
            for r, want in ref["ref"].items():
                sl = slice(cu[b] + r * cfg.block, cu[b] + min(L, (r + 1) * cfg.block))
                check_attention(out[sl, h], want, cfg.dtype, f"packed seq {b} h{h} row {r}")
            nchecked += 1
        r0 += rows_b
    print(f"[packed {name}] {nchecked} heads of {sum(1 for L in lens if L)} sequences bit-exact", flush=True)


def run_layer(F, pool, name, cfg):
    gen = LayerGen(cfg)
    reps = representatives(gen)
    dense = name == "llama8b_32k"
    # the oracle starts on every head at once, beside the GPU work
    jobs = [pool.submit(oracle_head, cfg, h, row_sample(cfg, h, h in reps), None,
                        [0, cfg.nb // 2, cfg.nb - 1] if dense and h in reps else ())
            for h in range(cfg.Hq)]
    print(f"[{name}] generating", flush=True)
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, q, k, v)
    outd = F.dense_attend(q, k, v, block=cfg.block) if dense else None
    torch.cuda.synchronize()
    gpu = gpu_plan_arrays(P, cfg)
    info = P.info()
    lists = P.lists()
    floor = O.floor_blocks(cfg.min_budget, cfg.block)
    for bh in range(cfg.B * cfg.Hq):
        list_properties(lists[bh], cfg.nb, floor)
    assert info.total_blocks == int(gpu["row_ptr"][-1])
    print(f"[{name}] density {info.total_blocks / info.dense_blocks:.4f}, "
          f"query-aware heads {info.query_aware_heads}; waiting for the oracle", flush=True)
    by_type = {}
    for fut in jobs:
        ref = fut.result()
        h = ref["h"]
        compare_full_head(name, ref, gpu, h)
        for r, want in ref["ref"].items():
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), want, cfg.dtype, f"{name} h{h} row {r}")
        for r, want in ref["refd"].items():
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(outd[0, h, sl].float().cpu().numpy(), want, cfg.dtype, f"dense h{h} row {r}")
        t = by_type.setdefault((ref["type"], ref["pattern"]), [0, 0])
        t[0] += 1
        t[1] += ref["blocks"]
    tri = cfg.nb * (cfg.nb + 1) // 2
    print(f"[{name}] all {cfg.Hq} heads bit-exact; (planted type, pattern): heads, density = " +
          ", ".join(f"{k}: {v[0]}, {v[1] / (v[0] * tri):.4f}" for k, v in sorted(by_type.items())), flush=True)
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
                                                          ("llama8b_128k", 8192, "flattened"),
                                                          ("glm9b_64k_bs64", 8192, "flattened"),
                                                          ("llama8b_128k", 0, "querywise"),
                                                          ("glm9b_64k_bs64", 0, "querywise")])
def test_full_size_plan_options(F, pool, name, max_budget, qa_selection):
    """The optional settings at full size: every row within the cap, every
    head's lists bit-exact with the oracle's plan under the same settings,
    two sampled rows of attention per head."""
    cfg = BY_NAME[name]
    gen = LayerGen(cfg)
    kw = dict(max_budget=max_budget, qa_selection=qa_selection)
    jobs = [pool.submit(oracle_head, cfg, h, row_sample(cfg, h, False), kw) for h in range(cfg.Hq)]
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget, **kw)
    out = F.attend(P, q, k, v)
    torch.cuda.synchronize()
    cap = O.cap_blocks(max_budget, cfg.block) or cfg.nb
    gpu = gpu_plan_arrays(P, cfg)
    lists = P.lists()
    floor = O.floor_blocks(cfg.min_budget, cfg.block)
    for bh in range(cfg.B * cfg.Hq):
        list_properties(lists[bh], cfg.nb, floor)
        assert max(len(x) for x in lists[bh]) <= cap
    for fut in jobs:
        ref = fut.result()
        h = ref["h"]
        compare_full_head(f"{name} cap {max_budget} {qa_selection}", ref, gpu, h)
        for r, want in ref["ref"].items():
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), want, cfg.dtype, f"{name} h{h} row {r}")
    print(f"[{name} cap {max_budget} {qa_selection}] all {cfg.Hq} heads bit-exact", flush=True)
    del q, k, v, out, P
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama8b_128k", "glm9b_64k_bs64"])
def test_full_size_token_mode_every_head(F, pool, name):
    """A full-size layer with token-granular vertical lines: every head's
    block lists, pattern, divergence and selected columns (colptr, colidx)
    bit-exact with the oracle's token-mode plan, two sampled rows of
    attention per head within tolerance."""
    cfg = BY_NAME[name]
    kw = dict(vs_granularity="token")
    jobs = [pool.submit(oracle_head, cfg, h, row_sample(cfg, h, False), kw) for h in range(cfg.Hq)]
    q, k, v = LayerGen(cfg).torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget, **kw)
    out = F.attend(P, q, k, v)
    torch.cuda.synchronize()
    pattern, djs, row_ptr, col_idx = P.copy_out()
    colptr, colidx = P.debug("colptr"), P.debug("colidx")
    nb, bs = cfg.nb, cfg.block
    with_cols = 0
    for fut in jobs:
        ref = fut.result()
        h = ref["h"]
        where = f"token {name} head {h} ({ref['type']})"
        assert int(pattern[h]) == ref["pattern"] and djs[h] == ref["D"], where
        np.testing.assert_array_equal(np.diff(row_ptr[h * nb: (h + 1) * nb + 1]), ref["counts"], err_msg=where)
        np.testing.assert_array_equal(col_idx[row_ptr[h * nb]: row_ptr[(h + 1) * nb]], ref["flat"], err_msg=where)
        cols = ref["cols"]
        ptr = np.searchsorted(cols, np.arange(nb + 1) * bs).astype(np.int32)
        np.testing.assert_array_equal(colptr[h], ptr, err_msg=where + ": colptr")
        np.testing.assert_array_equal(colidx[h][: ptr[-1]], cols, err_msg=where + ": colidx")
        with_cols += int(cols.size > 0)
        for r, want in ref["ref"].items():
            sl = slice(r * bs, (r + 1) * bs)
            check_attention(out[0, h, sl].float().cpu().numpy(), want, cfg.dtype, f"{where} row {r}")
    print(f"[token {name}] all {cfg.Hq} heads bit-exact, {with_cols} with token columns", flush=True)
