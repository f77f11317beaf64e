"""GPU parity of the HIP path (through the C ABI) with the CPU oracle on
seeded inputs small enough for the oracle to run on every head and row:
pattern choices, divergences, block lists and every selection intermediate
bit-exact; attention outputs within max-abs 2e-2 / mean-abs 2e-3 (bf16) or
1e-4 (fp32) of the float64 oracle."""
import numpy as np
import pytest

import oracle as O
from synth import BY_NAME, LayerGen
from tests._parity import check_attention, compare_head, list_properties

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_long_context_last_amd as F
    from sparse_long_context_last_amd import _lib
    _lib.load()
    return F


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def run_and_compare(F, cfg, q, k, v, attention=True, dense=True):
    dt = cfg.dtype
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    P = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    dbg = {it: P.debug(it) for it in ("qbar", "kbar", "rowmax", "rowsum", "colsum", "diagsum",
                                      "atrue", "ahat")}
    pattern, djs, _, _ = P.copy_out()
    lists = P.lists()
    out = F.attend(P, qd, kd, vd) if attention else None
    outd = F.dense_attend(qd, kd, vd, block=cfg.block) if dense else None
    torch.cuda.synchronize()
    B, Hq = q.shape[0], q.shape[1]
    group = Hq // k.shape[1]
    plans = {}
    for b in range(B):
        for kv in range(k.shape[1]):
            np.testing.assert_array_equal(dbg["kbar"][b * k.shape[1] + kv], O.pool_mean(k[b, kv], cfg.block))
        for h in range(Hq):
            bh = b * Hq + h
            hp = O.plan_head(q[b, h], k[b, h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
            compare_head(P, dbg, pattern, djs, lists, bh, hp)
            list_properties(lists[bh], cfg.nb, O.floor_blocks(cfg.min_budget, cfg.block))
            plans[bh] = hp
            if attention:
                ref = O.attend_head(q[b, h], k[b, h // group], v[b, h // group], hp.mask, cfg.block)
                check_attention(out[b, h].float().cpu().numpy(), ref, dt, f"sparse b{b} h{h}")
            if dense:
                refd = O.attend_head(q[b, h], k[b, h // group], v[b, h // group], O.dense_mask(cfg.nb), cfg.block)
                check_attention(outd[b, h].float().cpu().numpy(), refd, dt, f"dense b{b} h{h}")
    info = P.info()
    assert info.total_blocks == sum(sum(len(x) for x in hp.lists) for hp in plans.values())
    assert info.query_aware_heads == sum(hp.pattern for hp in plans.values())
    return P, plans, out, outd


SMALL = {
    # the tiny fp32 layer in full (one head of each planted type)
    "tiny_fp32_4k": BY_NAME["tiny_fp32_4k"],
    # Llama-shaped GQA 4:1, bf16, 16 blocks
    "gqa_bf16_2k": BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=2048, mix=(0.25, 0.25, 0.25, 0.25)),
    # 9 blocks: the score kernel's last 256-key chunk is half full
    "ragged_bf16_1152": BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, N=1152, min_budget=256,
                                                      explicit_types=("V", "S", "QA", "N")),
    # block 128, 9 blocks, two batches of GQA 2:1 (head orders and row pairs across sequences)
    "gqa_bf16_1152_b2": BY_NAME["llama8b_32k"].with_(B=2, Hq=4, Hkv=2, N=1152, min_budget=256,
                                                      explicit_types=("N", "QA", "V", "S")),
    # block 64, 17 blocks, two batches
    "bs64_bf16_1088_b2": BY_NAME["glm9b_64k_bs64"].with_(B=2, Hq=4, Hkv=2, N=1088, min_budget=256,
                                                          explicit_types=("QA", "V", "S", "N")),
    # fp32 at block 64
    "bs64_fp32_1024": BY_NAME["tiny_fp32_4k"].with_(N=1024, block=64, min_budget=128),
    # head dim 64: bf16 GQA 4:1 at block 128, bf16 block 64 with two batches, fp32 at both blocks
    "d64_gqa_bf16_2k": BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=2048, d=64, mix=(0.25, 0.25, 0.25, 0.25)),
    "d64_bs64_bf16_1088_b2": BY_NAME["glm9b_64k_bs64"].with_(B=2, Hq=4, Hkv=2, N=1088, d=64, min_budget=256,
                                                              explicit_types=("QA", "V", "S", "N")),
    "d64_fp32_1024": BY_NAME["tiny_fp32_4k"].with_(N=1024, d=64),
    "d64_bs64_fp32_704": BY_NAME["tiny_fp32_4k"].with_(N=704, d=64, block=64, min_budget=128),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(F, name):
    cfg = SMALL[name]
    q, k, v = LayerGen(cfg).numpy_layer()
    run_and_compare(F, cfg, q, k, v)


def test_probes_match_oracle(F):
    rng = np.random.default_rng(0)
    x = np.concatenate([np.linspace(-100, 0, 200_001, dtype=np.float32),
                        -np.abs(rng.standard_normal(50_000).astype(np.float32)) * 60,
                        np.array([-100.5, -np.inf, 0.0, -0.0], np.float32)])
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty_like(xd)
    from sparse_long_context_last_amd import _lib
    lib = _lib.load()
    s = torch.cuda.current_stream().cuda_stream
    _lib.check(lib.fp_probe_exp2(xd.data_ptr(), yd.data_ptr(), x.size, s), "probe")
    np.testing.assert_array_equal(yd.cpu().numpy(), O.exp2_c(x))
    z = np.concatenate([np.exp(rng.uniform(-700, 700, 100_000)), rng.uniform(0, 2, 100_000),
                        [0.5, 1.0, 2.0, 1e-300]])
    zd = torch.from_numpy(z).cuda()
    wd = torch.empty_like(zd)
    _lib.check(lib.fp_probe_ln(zd.data_ptr(), wd.data_ptr(), z.size, s), "probe")
    np.testing.assert_array_equal(wd.cpu().numpy(), O.ln_c(z))
    sq = np.concatenate([rng.uniform(0, np.log(2), 200_000), rng.uniform(0, 1e-6, 50_000),
                         np.exp(rng.uniform(-700, 700, 50_000)), [0.0, 1.0, 2.0]])
    sd = torch.from_numpy(sq).cuda()
    rd = torch.empty_like(sd)
    _lib.check(lib.fp_probe_sqrt(sd.data_ptr(), rd.data_ptr(), sq.size, s), "probe")
    np.testing.assert_array_equal(rd.cpu().numpy(), np.sqrt(sq))


def test_gamma_one_equals_dense(F):
    cfg = SMALL["gqa_bf16_2k"].with_(gamma=1.0)
    q, k, v = LayerGen(cfg).numpy_layer()
    P, plans, out, outd = run_and_compare(F, cfg, q, k, v)
    assert P.info().total_blocks == P.info().dense_blocks
    # the same attention computed by the sparse kernel over full lists and by
    # the dense kernel (another tile schedule): equal to bf16 rounding
    check_attention(out.float().cpu().numpy(), outd.double().cpu().numpy(), "bf16", "sparse vs dense")
    # the fp32 kernel serves both paths with one schedule: bit for bit
    cfg32 = BY_NAME["tiny_fp32_4k"].with_(N=1024, gamma=1.0)
    q, k, v = LayerGen(cfg32).numpy_layer()
    qd, kd, vd = to_dev(q, "fp32"), to_dev(k, "fp32"), to_dev(v, "fp32")
    P32 = F.plan(qd, kd, block=128, gamma=1.0, tau=cfg32.tau, min_budget=cfg32.min_budget)
    assert torch.equal(F.attend(P32, qd, kd, vd), F.dense_attend(qd, kd, vd, block=128))


def test_tau_extremes_and_budget(F):
    base = SMALL["gqa_bf16_2k"]
    q, k, v = LayerGen(base).numpy_layer()
    _, plans, _, _ = run_and_compare(F, base.with_(tau=0.0), q, k, v, dense=False)
    assert all(hp.pattern == O.VERTICAL_SLASH for hp in plans.values())
    _, plans, _, _ = run_and_compare(F, base.with_(tau=0.84), q, k, v, dense=False)
    assert all(hp.pattern == O.QUERY_AWARE for hp in plans.values())
    P, _, _, _ = run_and_compare(F, base.with_(min_budget=base.N), q, k, v, dense=False)
    assert P.info().total_blocks == P.info().dense_blocks
    run_and_compare(F, base.with_(gamma=0.5, min_budget=0), q, k, v, dense=False)


def test_single_block_and_zero_inputs(F):
    cfg = SMALL["ragged_bf16_1152"].with_(N=128)
    q, k, v = LayerGen(cfg).numpy_layer()
    P, plans, _, _ = run_and_compare(F, cfg, q, k, v)
    assert all(hp.D == 0.0 for hp in plans.values())
    # all-zero queries and keys: uniform attention, every selection decided by
    # the index tie-break
    cfg = SMALL["ragged_bf16_1152"].with_(gamma=0.6, min_budget=0)
    z = np.zeros((1, cfg.Hq, cfg.N, cfg.d), np.float32)
    zk = np.zeros((1, cfg.Hkv, cfg.N, cfg.d), np.float32)
    v = LayerGen(cfg).numpy_layer()[2]
    run_and_compare(F, cfg, z, zk, v)


def test_plans_are_deterministic(F):
    cfg = SMALL["gqa_bf16_2k"]
    q, k, v = LayerGen(cfg).numpy_layer()
    qd, kd = to_dev(q, "bf16"), to_dev(k, "bf16")
    a = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    b = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    for x, y in zip(a.copy_out(), b.copy_out()):
        np.testing.assert_array_equal(x, y)
    for it in ("colsum", "diagsum", "ahat"):
        np.testing.assert_array_equal(a.debug(it), b.debug(it))


def test_empty_problem_on_device(F):
    cfg = SMALL["gqa_bf16_2k"]
    q = torch.zeros((0, cfg.Hq, cfg.N, cfg.d), device="cuda", dtype=torch.bfloat16)
    k = torch.zeros((0, cfg.Hkv, cfg.N, cfg.d), device="cuda", dtype=torch.bfloat16)
    P = F.plan(q, k, block=128)
    assert P.info().total_blocks == 0
    out = F.attend(P, q, k, k)
    assert out.shape == q.shape


def run_capped(F, cfg, q, k, v, max_budget, qa_selection="flattened"):
    """Plan with the optional settings; lists bit-exact with the oracle's,
    attention within tolerance; returns how many rows the cap shortened."""
    dt = cfg.dtype
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    P = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
               max_budget=max_budget, qa_selection=qa_selection)
    out = F.attend(P, qd, kd, vd)
    torch.cuda.synchronize()
    assert P.info().max_budget == max_budget
    assert P.info().qa_selection == (1 if qa_selection == "querywise" else 0)
    pattern, djs, _, _ = P.copy_out()
    lists = P.lists()
    group = cfg.Hq // cfg.Hkv
    cap = O.cap_blocks(max_budget, cfg.block) or cfg.nb
    capped_rows = 0
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            bh = b * cfg.Hq + h
            hp = O.plan_head(q[b, h], k[b, h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, max_budget,
                             qa_selection)
            assert int(pattern[bh]) == hp.pattern and djs[bh] == hp.D
            for r in range(cfg.nb):
                assert np.array_equal(lists[bh][r], hp.lists[r]), (bh, r, lists[bh][r][:12], hp.lists[r][:12])
                assert len(hp.lists[r]) <= cap
            capped_rows += sum(1 for x in O.plan_head(q[b, h], k[b, h // group], cfg.block, cfg.gamma, cfg.tau,
                                                      cfg.min_budget, 0, qa_selection).lists if len(x) > cap)
            ref = O.attend_head(q[b, h], k[b, h // group], v[b, h // group], hp.mask, cfg.block)
            check_attention(out[b, h].float().cpu().numpy(), ref, dt, f"capped b{b} h{h}")
    return capped_rows


@pytest.mark.parametrize("name,max_budget", [("gqa_bf16_2k", 1024), ("gqa_bf16_2k", 1536),
                                             ("bs64_bf16_1088_b2", 512), ("tiny_fp32_4k", 2048)])
def test_max_budget_parity(F, name, max_budget):
    cfg = SMALL[name]
    q, k, v = LayerGen(cfg).numpy_layer()
    assert run_capped(F, cfg, q, k, v, max_budget) > 0     # the cap was exercised


def test_max_budget_with_gamma_one_and_ties(F):
    cfg = SMALL["ragged_bf16_1152"].with_(gamma=1.0)
    q, k, v = LayerGen(cfg).numpy_layer()
    assert run_capped(F, cfg, q, k, v, 512) > 0
    z = np.zeros((1, cfg.Hq, cfg.N, cfg.d), np.float32)            # every score ties
    zk = np.zeros((1, cfg.Hkv, cfg.N, cfg.d), np.float32)
    run_capped(F, cfg.with_(gamma=0.7), z, zk, v, 384)


@pytest.mark.parametrize("name,max_budget", [("gqa_bf16_2k", 0), ("tiny_fp32_4k", 0), ("bs64_bf16_1088_b2", 0),
                                             ("ragged_bf16_1152", 0), ("gqa_bf16_2k", 1024)])
def test_querywise_selection_parity(F, name, max_budget):
    cfg = SMALL[name]
    q, k, v = LayerGen(cfg).numpy_layer()
    run_capped(F, cfg, q, k, v, max_budget, qa_selection="querywise")


def test_querywise_all_query_aware_and_ties(F):
    base = SMALL["gqa_bf16_2k"]
    q, k, v = LayerGen(base).numpy_layer()
    run_capped(F, base.with_(tau=0.84, gamma=0.8, min_budget=0), q, k, v, 0, qa_selection="querywise")
    cfg = SMALL["ragged_bf16_1152"].with_(gamma=0.6, min_budget=0, tau=0.84)
    z = np.zeros((1, cfg.Hq, cfg.N, cfg.d), np.float32)            # uniform rows: pure tie-break
    zk = np.zeros((1, cfg.Hkv, cfg.N, cfg.d), np.float32)
    run_capped(F, cfg, z, zk, LayerGen(cfg).numpy_layer()[2], 0, qa_selection="querywise")


def _wide_bf16(rng, shape, emin, emax):
    """bf16-representable values with random signs, 7-bit mantissas and
    exponents uniform in [emin, emax], as float32."""
    e = rng.integers(emin, emax + 1, size=shape)
    m = rng.integers(0, 128, size=shape)
    s = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    return (s * (1.0 + m / 128.0) * np.exp2(e.astype(np.float64))).astype(np.float32)


@pytest.mark.parametrize("block", [128, 64])
def test_wide_range_bf16_scores(F, block):
    """bf16 inputs over a wide exponent range (every third query row and every
    fifth key row with exponents in [-75, -64], so about 5 % of the last-block
    dot products are denormal): the last-block statistics, divergences and
    lists stay bit-exact."""
    cfg = BY_NAME["llama8b_32k"].with_(Hq=2, Hkv=1, N=640, block=block, min_budget=256, gamma=0.9)
    rng = np.random.default_rng(7)
    q = _wide_bf16(rng, (1, cfg.Hq, cfg.N, cfg.d), -40, 6)
    k = _wide_bf16(rng, (1, cfg.Hkv, cfg.N, cfg.d), -40, 6)
    q[:, :, ::3, :] = _wide_bf16(rng, q[:, :, ::3, :].shape, -75, -64)
    k[:, :, ::5, :] = _wide_bf16(rng, k[:, :, ::5, :].shape, -75, -64)
    v = rng.standard_normal((1, cfg.Hkv, cfg.N, cfg.d)).astype(np.float32)
    run_and_compare(F, cfg, q, k, v, attention=False, dense=False)


def test_plan_log_lines_match_the_plan(F, monkeypatch, capfd):
    """FP_LOG=1: one line for the plan and one per head whose pattern,
    divergence and block count agree with the plan's own copy."""
    import re
    cfg = SMALL["gqa_bf16_2k"]
    q, k, _ = LayerGen(cfg).numpy_layer()
    monkeypatch.setenv("FP_LOG", "1")
    P = F.plan(to_dev(q, "bf16"), to_dev(k, "bf16"), block=cfg.block, gamma=cfg.gamma, tau=cfg.tau,
               min_budget=cfg.min_budget)
    monkeypatch.delenv("FP_LOG")
    err = capfd.readouterr().err
    pattern, djs, row_ptr, _ = P.copy_out()
    lines = [l for l in err.splitlines() if l.startswith("[fp_prefill]   seq")]
    assert len(lines) == cfg.Hq and "[fp_prefill] plan: 1 sequence(s), Hq 8, Hkv 2" in err
    tri = cfg.nb * (cfg.nb + 1) // 2
    for h, line in enumerate(lines):
        m = re.search(r"head (\d+): (\S+)\s+D (\S+) blocks (\d+) / (\d+)", line)
        assert int(m.group(1)) == h
        assert m.group(2) == ("query-aware" if pattern[h] == O.QUERY_AWARE else "vertical-slash")
        assert abs(float(m.group(3)) - djs[h]) <= 5e-7
        assert int(m.group(4)) == row_ptr[(h + 1) * cfg.nb] - row_ptr[h * cfg.nb] and int(m.group(5)) == tri
