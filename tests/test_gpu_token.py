"""GPU parity of the token-granular vertical-slash mode (vs_granularity =
"token"): block lists (slash blocks, floor, cap), the compacted column lists
and the attention over full blocks plus gathered columns, against the
oracle's token-level definition."""
import numpy as np
import pytest

import oracle as O
from synth import BY_NAME, LayerGen
from tests._parity import check_attention, list_properties

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


def oracle_cols(hp, bs):
    """colptr / colidx of one head as the plan stores them."""
    N = hp.stats.c.shape[0]
    nb = -(-N // bs)
    cols = np.zeros(N, bool) if hp.cols is None else hp.cols
    idx = np.nonzero(cols)[0]
    ptr = np.array([np.count_nonzero(idx < kb * bs) for kb in range(nb + 1)], np.int32)
    return ptr, idx.astype(np.int32)


def check_token_layer(F, cfg, q, k, v, N, max_budget=0, rows=None):
    dt = cfg.dtype
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    P = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
               max_budget=max_budget, vs_granularity="token")
    out = F.attend(P, qd, kd, vd)
    torch.cuda.synchronize()
    assert P.info().vs_granularity == 1
    pattern, djs, _, _ = P.copy_out()
    lists = P.lists()
    colptr, colidx = P.debug("colptr"), P.debug("colidx")
    nb = -(-N // cfg.block)
    group = cfg.Hq // cfg.Hkv
    n_vs_with_cols = 0
    heads = range(cfg.B * cfg.Hq) if rows is None else rows.keys()
    for bh in heads:
        b, h = divmod(bh, cfg.Hq)
        hp = O.plan_head(q[b, h], k[b, h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, max_budget,
                         vs_granularity="token")
        assert int(pattern[bh]) == hp.pattern and djs[bh] == hp.D
        for r in range(nb):
            assert np.array_equal(lists[bh][r], hp.lists[r]), (bh, r, lists[bh][r][:12], hp.lists[r][:12])
        list_properties(lists[bh], nb, O.floor_blocks(cfg.min_budget, cfg.block))
        ptr, idx = oracle_cols(hp, cfg.block)
        np.testing.assert_array_equal(colptr[bh], ptr)
        np.testing.assert_array_equal(colidx[bh][: ptr[-1]], idx)
        n_vs_with_cols += int(ptr[-1] > 0)
        sel = range(nb) if rows is None else rows[bh]
        ref = O.attend_rows(q[b, h], k[b, h // group], v[b, h // group], hp.mask, cfg.block, sel, hp.cols)
        for r in sel:
            sl = slice(r * cfg.block, min(N, (r + 1) * cfg.block))
            check_attention(out[b, h, sl].float().cpu().numpy(), ref[r], dt, f"token b{b} h{h} row {r}")
    return n_vs_with_cols


SMALL = {
    "gqa_bf16_2k": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=2048, mix=(0.5, 0.25, 0.25, 0.0)), 2048),
    "ragged_bf16_1100": (BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, N=1152, min_budget=256,
                                                      explicit_types=("V", "V", "QA", "S")), 1100),
    "bs64_bf16_b2": (BY_NAME["glm9b_64k_bs64"].with_(B=2, Hq=4, Hkv=2, N=1088, min_budget=256,
                                                     explicit_types=("V", "V", "S", "QA")), 1088),
    "fp32_1024": (BY_NAME["tiny_fp32_4k"].with_(N=1024, explicit_types=("V", "V", "S", "QA")), 1024),
    "d64_bf16_2k": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=2048, d=64, mix=(0.5, 0.25, 0.25, 0.0)), 2048),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_token_mode_small_layers(F, name):
    cfg, N = SMALL[name]
    q, k, v = (x[:, :, :N] for x in LayerGen(cfg).numpy_layer())
    assert check_token_layer(F, cfg, q, k, v, N) > 0       # some vertical-slash head had columns


def test_token_mode_with_cap_and_tau_zero(F):
    cfg, N = SMALL["gqa_bf16_2k"]
    q, k, v = LayerGen(cfg).numpy_layer()
    check_token_layer(F, cfg.with_(tau=0.0, min_budget=256), q, k, v, N, max_budget=512)


def test_token_mode_varlen(F):
    cfg = BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, explicit_types=("V", "V", "S", "QA"))
    lens = [900, 0, 2048, 130]
    seqs = []
    for b, L in enumerate(lens):
        q, k, v = LayerGen(cfg.with_(N=max(128, -(-L // 128) * 128), seed=cfg.seed + 3 * b)).numpy_layer()
        seqs.append((q[0, :, :L], k[0, :, :L], v[0, :, :L]))
    cat = [np.concatenate([s[i].transpose(1, 0, 2) for s in seqs], axis=0) for i in range(3)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qd, kd, vd = (dev(x, "bf16") for x in cat)
    P = F.plan_varlen(qd, kd, cu, block=128, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
                      vs_granularity="token")
    out = F.attend(P, qd, kd, vd).float().cpu().numpy()
    lists = P.lists()
    cps = P.debug_seqs("colptr")
    for b, (q, k, v) in enumerate(seqs):
        if lens[b] == 0:
            continue
        for h in range(cfg.Hq):
            hp = O.plan_head(q[h], k[0], 128, cfg.gamma, cfg.tau, cfg.min_budget, vs_granularity="token")
            for r, x in enumerate(hp.lists):
                assert np.array_equal(lists[b * cfg.Hq + h][r], x), (b, h, r)
            np.testing.assert_array_equal(cps[b][h], oracle_cols(hp, 128)[0])
            ref = O.attend_head(q[h], k[0], v[0], hp.mask, 128, hp.cols)
            check_attention(out[cu[b]:cu[b + 1], h], ref, "bf16", f"seq {b} h{h}")


def test_token_mode_full_size_128k(F):
    """The 128k layer in token mode: sampled vertical heads (lists, columns,
    rows of attention) against the oracle; the other heads' plans keep their
    block-mode lists."""
    cfg = BY_NAME["llama8b_128k"]
    gen = LayerGen(cfg)
    q, k, v = gen.torch_layer("cuda")
    P = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
               vs_granularity="token")
    out = F.attend(P, q, k, v)
    Pb = F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    torch.cuda.synchronize()
    pattern = P.copy_out()[0]
    lists, lists_b = P.lists(), Pb.lists()
    colptr, colidx = P.debug("colptr"), P.debug("colidx")
    for h in range(cfg.Hq):
        if pattern[h] == O.QUERY_AWARE:
            assert all(np.array_equal(x, y) for x, y in zip(lists[h], lists_b[h]))
    info, info_b = P.info(), Pb.info()
    print(f"[token 128k] blocks {info.total_blocks} (block mode {info_b.total_blocks})", flush=True)
    assert info.total_blocks < info_b.total_blocks
    rng = np.random.default_rng(3)
    vs_heads = [h for h in range(cfg.Hq) if pattern[h] == O.VERTICAL_SLASH][:2]
    for h in vs_heads:
        qh, kh, vh = gen.q_head(0, h), gen.k_head(0, h // cfg.group), gen.v_head(0, h // cfg.group)
        hp = O.plan_head(qh, kh, cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, vs_granularity="token")
        for r in range(cfg.nb):
            assert np.array_equal(lists[h][r], hp.lists[r]), (h, r)
        ptr, idx = oracle_cols(hp, cfg.block)
        np.testing.assert_array_equal(colptr[h], ptr)
        np.testing.assert_array_equal(colidx[h][: ptr[-1]], idx)
        rows = sorted(set([0, cfg.nb - 1] + rng.choice(cfg.nb, 3, replace=False).tolist()))
        ref = O.attend_rows(qh, kh, vh, hp.mask, cfg.block, rows, hp.cols)
        for r in rows:
            sl = slice(r * cfg.block, (r + 1) * cfg.block)
            check_attention(out[0, h, sl].float().cpu().numpy(), ref[r], "bf16", f"128k token h{h} row {r}")
    del q, k, v, out, P, Pb
    torch.cuda.empty_cache()
