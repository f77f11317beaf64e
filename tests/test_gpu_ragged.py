"""GPU parity for sequences whose length is not a multiple of the block and
for packed batches of sequences of different lengths ([T, H, d] with
cu_seqlens), through the C ABI, against the CPU oracle run per sequence and
head: every selection intermediate, divergence, pattern and block list
bit-exact; attention within the dtype's tolerance."""
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
    return F


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def layer(cfg, N, seed_shift=0):
    """Seeded inputs of cfg's shape cut to N tokens (generated at a whole
    number of 128-token segments)."""
    n_gen = max(128, -(-N // 128) * 128)
    q, k, v = LayerGen(cfg.with_(N=n_gen, seed=cfg.seed + seed_shift)).numpy_layer()
    return q[:, :, :N], k[:, :, :N], v[:, :, :N]


RAGGED = {
    # GQA 4:1 bf16, 8 blocks of 128 with a 104-token last block
    "gqa_bf16_1000": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, mix=(0.25, 0.25, 0.25, 0.25)), 1000),
    # block 64, two sequences, one token in the last block
    "bs64_bf16_1089_b2": (BY_NAME["glm9b_64k_bs64"].with_(B=2, Hq=4, Hkv=2, min_budget=256,
                                                          explicit_types=("QA", "V", "S", "N")), 1089),
    # shorter than one block: a single partial block, 100 representative rows
    "short_bf16_100": (BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, explicit_types=("V", "S", "QA", "N")), 100),
    # a single token
    "one_token_bf16": (BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=1, explicit_types=("V", "S", "QA", "N")), 1),
    # fp32, block 64, 700 tokens
    "fp32_bs64_700": (BY_NAME["tiny_fp32_4k"].with_(block=64, min_budget=128), 700),
    # head dim 64: bf16 at block 64 with two sequences, fp32 at block 128
    "d64_bs64_bf16_1000_b2": (BY_NAME["glm9b_64k_bs64"].with_(B=2, Hq=4, Hkv=2, d=64, min_budget=256,
                                                              explicit_types=("QA", "V", "S", "N")), 1000),
    "d64_fp32_900": (BY_NAME["tiny_fp32_4k"].with_(d=64, min_budget=256), 900),
}


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_layer_parity(F, name):
    cfg, N = RAGGED[name]
    check_layer(F, cfg, N, name)


def check_layer(F, cfg, N, name=""):
    """Plan, sparse and dense attention of cfg's seeded inputs cut to N
    tokens against the oracle: every head's intermediates and lists bit-exact,
    outputs within tolerance."""
    q, k, v = layer(cfg, N)
    dt = tdt(cfg.dtype)
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (q, k, v))
    P = F.plan(qd, kd, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    dbg = {it: P.debug(it) for it in ("qbar", "kbar", "rowmax", "rowsum", "colsum", "diagsum", "atrue", "ahat")}
    pattern, djs, _, _ = P.copy_out()
    lists = P.lists()
    out = F.attend(P, qd, kd, vd)
    outd = F.dense_attend(qd, kd, vd, block=cfg.block)
    torch.cuda.synchronize()
    nb = -(-N // cfg.block)
    info = P.info()
    assert info.nb == nb and info.rows == cfg.B * cfg.Hq * nb
    group = cfg.Hq // cfg.Hkv
    total = 0
    for b in range(cfg.B):
        for kv in range(cfg.Hkv):
            np.testing.assert_array_equal(dbg["kbar"][b * cfg.Hkv + kv], O.pool_mean(k[b, kv], cfg.block))
        for h in range(cfg.Hq):
            bh = b * cfg.Hq + h
            hp = O.plan_head(q[b, h], k[b, h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
            compare_head(P, dbg, pattern, djs, lists, bh, hp)
            list_properties(lists[bh], nb, O.floor_blocks(cfg.min_budget, cfg.block))
            total += sum(len(x) for x in hp.lists)
            ref = O.attend_head(q[b, h], k[b, h // group], v[b, h // group], hp.mask, cfg.block)
            check_attention(out[b, h].float().cpu().numpy(), ref, cfg.dtype, f"{name} sparse b{b} h{h}")
            refd = O.attend_head(q[b, h], k[b, h // group], v[b, h // group], O.dense_mask(nb), cfg.block)
            check_attention(outd[b, h].float().cpu().numpy(), refd, cfg.dtype, f"{name} dense b{b} h{h}")
    assert info.total_blocks == total


def packed(cfg, lens):
    """Packed [T, H, d] tensors of sequences with their own seeds, plus the
    per-sequence [H, L, d] arrays the oracle reads."""
    seqs = [layer(cfg.with_(B=1), max(L, 1), seed_shift=7 * b) for b, L in enumerate(lens)]
    seqs = [(q[0, :, :L], k[0, :, :L], v[0, :, :L]) for (q, k, v), L in zip(seqs, lens)]
    cat = [np.concatenate([s[i].transpose(1, 0, 2) for s in seqs], axis=0) for i in range(3)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return seqs, cat, cu


VARLEN = {
    "gqa_bf16_mixed": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, mix=(0.25, 0.25, 0.25, 0.25)),
                       [1000, 0, 257, 2048, 64, 1]),
    "bs64_bf16_mixed": (BY_NAME["glm9b_64k_bs64"].with_(Hq=4, Hkv=2, min_budget=256,
                                                        explicit_types=("QA", "V", "S", "N")), [1089, 130, 64]),
    "fp32_mixed": (BY_NAME["tiny_fp32_4k"].with_(min_budget=256), [300, 1024, 5]),
    "d64_bf16_mixed": (BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, d=64, mix=(0.25, 0.25, 0.25, 0.25)),
                       [700, 0, 2048, 65]),
}


@pytest.mark.parametrize("name", list(VARLEN))
def test_varlen_parity(F, name):
    cfg, lens = VARLEN[name]
    check_packed(F, cfg, lens, name)


def check_packed(F, cfg, lens, name=""):
    """A packed batch of sequences with their own seeds against the oracle:
    every head of every sequence bit-exact, sparse and dense outputs within
    tolerance."""
    seqs, (qc, kc, vc), cu = packed(cfg, lens)
    dt = tdt(cfg.dtype)
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (qc, kc, vc))
    P = F.plan_varlen(qd, kd, cu, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    dbg_seq = {it: P.debug_seqs(it) for it in ("qbar", "rowmax", "rowsum", "colsum", "diagsum", "atrue", "ahat")}
    pattern, djs, _, _ = P.copy_out()
    lists = P.lists()
    out = F.attend(P, qd, kd, vd).float().cpu().numpy()
    outd = F.dense_attend_varlen(qd, kd, vd, cu, block=cfg.block).float().cpu().numpy()
    info = P.info()
    assert info.layout == 1 and info.tokens == cu[-1] and info.B == len(lens) and info.N == max(lens)
    group = cfg.Hq // cfg.Hkv
    total = 0
    for b, (q, k, v) in enumerate(seqs):
        L = lens[b]
        if L == 0:
            assert all(len(lists[b * cfg.Hq + h]) == 0 for h in range(cfg.Hq))
            assert not pattern[b * cfg.Hq:(b + 1) * cfg.Hq].any()
            continue
        nb = -(-L // cfg.block)
        dbg = {it: np.concatenate([np.zeros((b * cfg.Hq,) + x[b].shape[1:], x[b].dtype), x[b]])
               for it, x in dbg_seq.items()}   # index by b * Hq + h
        for h in range(cfg.Hq):
            bh = b * cfg.Hq + h
            hp = O.plan_head(q[h], k[h // group], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
            compare_head(P, dbg, pattern, djs, lists, bh, hp)
            total += sum(len(x) for x in hp.lists)
            ref = O.attend_head(q[h], k[h // group], v[h // group], hp.mask, cfg.block)
            check_attention(out[cu[b]:cu[b + 1], h], ref, cfg.dtype, f"{name} seq {b} h{h}")
            refd = O.attend_head(q[h], k[h // group], v[h // group], O.dense_mask(nb), cfg.block)
            check_attention(outd[cu[b]:cu[b + 1], h], refd, cfg.dtype, f"{name} dense seq {b} h{h}")
    assert info.total_blocks == total


def test_varlen_equal_lengths_match_the_batched_layout(F):
    """Packed sequences of one length plan and attend exactly like the
    [B, H, N, d] layout: identical lists and bit-identical outputs."""
    cfg = BY_NAME["llama8b_32k"].with_(B=3, Hq=8, Hkv=2, mix=(0.25, 0.25, 0.25, 0.25))
    N = 777
    q, k, v = layer(cfg, N)
    dt = torch.bfloat16
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (q, k, v))
    P = F.plan(qd, kd, block=128, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    out = F.attend(P, qd, kd, vd)
    pk = [x.permute(0, 2, 1, 3).reshape(cfg.B * N, x.shape[1], 128).contiguous() for x in (qd, kd, vd)]
    cu = np.arange(cfg.B + 1, dtype=np.int32) * N
    Pv = F.plan_varlen(pk[0], pk[1], cu, block=128, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    outv = F.attend(Pv, *pk)
    torch.cuda.synchronize()
    a, b = P.copy_out(), Pv.copy_out()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert torch.equal(out.permute(0, 2, 1, 3).reshape(cfg.B * N, cfg.Hq, 128), outv)


def test_varlen_with_options(F):
    cfg, lens = VARLEN["gqa_bf16_mixed"]
    seqs, (qc, kc, vc), cu = packed(cfg, lens)
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16) for x in (qc, kc, vc))
    P = F.plan_varlen(qd, kd, cu, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=256,
                      max_budget=512, qa_selection="querywise")
    lists = P.lists()
    out = F.attend(P, qd, kd, vd).float().cpu().numpy()
    group = cfg.Hq // cfg.Hkv
    for b, (q, k, v) in enumerate(seqs):
        if lens[b] == 0:
            continue
        for h in range(cfg.Hq):
            hp = O.plan_head(q[h], k[h // group], cfg.block, cfg.gamma, cfg.tau, 256, 512, "querywise")
            for r, x in enumerate(hp.lists):
                assert np.array_equal(lists[b * cfg.Hq + h][r], x), (b, h, r)
                assert len(x) <= 4
            ref = O.attend_head(q[h], k[h // group], v[h // group], hp.mask, cfg.block)
            check_attention(out[cu[b]:cu[b + 1], h], ref, "bf16", f"seq {b} h{h}")
