"""Pins of the oracle's attention half and of whole-head plans (no GPU):
gamma = 1 and a budget >= N reproduce full causal attention (torch's
scaled-dot-product attention in float64), arbitrary block masks match a
per-token brute force, and the divergence threshold behaves as the pages'
ablation describes (tau = 0 switches query-aware off)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import BY_NAME, LayerGen

F32 = np.float32


def sdpa_causal(q, k, v):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    return out[0, 0].numpy()


@pytest.fixture(scope="module")
def small_layer():
    cfg = BY_NAME["tiny_fp32_4k"].with_(N=1024)
    gen = LayerGen(cfg)
    q, k, v = gen.numpy_layer()
    return cfg, q, k, v


def test_gamma_one_is_full_causal_attention(small_layer):
    cfg, q, k, v = small_layer
    for h in range(cfg.Hq):
        P = O.plan_head(q[0, h], k[0, h], cfg.block, 1.0, cfg.tau, cfg.min_budget)
        assert np.array_equal(P.mask, O.dense_mask(cfg.nb))
        out = O.attend_head(q[0, h], k[0, h], v[0, h], P.mask, cfg.block)
        np.testing.assert_allclose(out, sdpa_causal(q[0, h], k[0, h], v[0, h]), rtol=0, atol=1e-12)


def test_budget_covering_sequence_is_full_attention(small_layer):
    cfg, q, k, v = small_layer
    P = O.plan_head(q[0, 0], k[0, 0], cfg.block, 0.5, cfg.tau, cfg.N)
    assert np.array_equal(P.mask, O.dense_mask(cfg.nb))


def brute_force_attention(q, k, v, mask, bs):
    N, d = q.shape
    out = np.zeros((N, v.shape[1]))
    for i in range(N):
        ws, acc = [], np.zeros(v.shape[1])
        keys = [j for j in range(i + 1) if mask[i // bs, j // bs]]
        s = [sum(float(q[i, t]) * float(k[j, t]) for t in range(d)) / math.sqrt(d) for j in keys]
        m = max(s)
        ws = [math.exp(x - m) for x in s]
        z = sum(ws)
        for w, j in zip(ws, keys):
            acc += (w / z) * v[j].astype(np.float64)
        out[i] = acc
    return out


@pytest.mark.parametrize("N,bs", [(1000, 128), (200, 64), (70, 128)])
def test_ragged_gamma_one_is_full_causal_attention(N, bs):
    cfg = BY_NAME["tiny_fp32_4k"].with_(N=1024)
    q, k, v = (x[0, 0, :N] for x in LayerGen(cfg).numpy_layer())
    P = O.plan_head(q, k, bs, 1.0, 0.1, 0)
    nb = -(-N // bs)
    assert np.array_equal(P.mask, O.dense_mask(nb)) and len(P.lists) == nb
    out = O.attend_head(q, k, v, P.mask, bs)
    assert out.shape == (N, 128)
    np.testing.assert_allclose(out, sdpa_causal(q, k, v), rtol=0, atol=1e-12)


def test_ragged_plan_lists_and_masked_attention():
    """A ragged sequence's plan keeps the floor and causality, and its
    attention equals the per-token brute force under the plan's mask."""
    rng = np.random.default_rng(23)
    bs, N, d = 8, 45, 16
    q = rng.standard_normal((N, d)).astype(F32)
    k = rng.standard_normal((N, d)).astype(F32)
    v = rng.standard_normal((N, d)).astype(F32)
    for tau in (0.0, 0.84):
        P = O.plan_head(q, k, bs, 0.6, tau, 2 * bs)
        nb = -(-N // bs)
        assert len(P.lists) == nb
        for qb, lst in enumerate(P.lists):
            assert len(lst) >= min(qb + 1, 2) and lst.max() <= qb
        np.testing.assert_allclose(O.attend_head(q, k, v, P.mask, bs),
                                   brute_force_attention(q, k, v, P.mask, bs), rtol=0, atol=1e-12)


def test_masked_attention_equals_per_token_brute_force():
    rng = np.random.default_rng(21)
    bs, nb, d = 8, 5, 16
    N = bs * nb
    q = rng.standard_normal((N, d)).astype(F32)
    k = rng.standard_normal((N, d)).astype(F32)
    v = rng.standard_normal((N, d)).astype(F32)
    mask = np.tril(rng.random((nb, nb)) < 0.5)
    mask = O.apply_floor(mask, 0, bs)
    got = O.attend_head(q, k, v, mask, bs)
    ref = brute_force_attention(q, k, v, mask, bs)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_tau_zero_disables_query_aware_and_large_tau_forces_it(small_layer):
    cfg, q, k, v = small_layer
    for h in range(cfg.Hq):
        P0 = O.plan_head(q[0, h], k[0, h], cfg.block, cfg.gamma, 0.0, cfg.min_budget)
        assert P0.pattern == O.VERTICAL_SLASH
        P1 = O.plan_head(q[0, h], k[0, h], cfg.block, cfg.gamma, 0.84, cfg.min_budget)
        assert P1.pattern == O.QUERY_AWARE          # D <= sqrt(ln 2) < 0.84


def test_planted_types_on_tiny_layer():
    """The planted vertical head falls back to vertical-slash (its pooled
    estimate misses the sink keys); the query-aware head keeps query-aware."""
    cfg = BY_NAME["tiny_fp32_4k"]
    gen = LayerGen(cfg)
    q, k, v = gen.numpy_layer()
    pats = []
    for h in range(cfg.Hq):
        P = O.plan_head(q[0, h], k[0, h], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
        pats.append(P.pattern)
        assert all(len(x) >= min(qb + 1, 8) for qb, x in enumerate(P.lists))
        sel_mass = None
        if P.sel_qa is not None:
            vals = O.tri_values(P.A).astype(np.float64)
            sel_mass = vals[P.sel_qa].sum() / vals.sum()
        else:
            sel_mass = P.stats.c[P.sel_v].astype(np.float64).sum() / P.stats.c.astype(np.float64).sum()
        assert sel_mass >= cfg.gamma - 1e-6
    assert pats[0] == O.VERTICAL_SLASH
    assert pats[2] == O.QUERY_AWARE


def test_constant_inputs_tie_break():
    """All-zero queries and keys: every score is 0, the attention is uniform
    and every selection is decided by the index tie-break."""
    bs, nb, d = 16, 6, 32
    N = bs * nb
    q = np.zeros((N, d), F32)
    k = np.zeros((N, d), F32)
    P = O.plan_head(q, k, bs, 0.5, 0.1, 0)
    assert P.D == 0.0 or P.pattern == O.QUERY_AWARE
    # the estimate is uniform per row; flattened ties resolve to the lowest
    # flat indices, i.e. the earliest rows
    assert P.pattern == O.QUERY_AWARE
    flat = np.nonzero(P.sel_qa)[0]
    assert flat.tolist() == list(range(len(flat)))
    # single block: the whole plan degenerates to the one diagonal block
    P1 = O.plan_head(q[:bs], k[:bs], bs, 0.95, 0.1, 0)
    assert P1.D == 0.0 and [x.tolist() for x in P1.lists] == [[0]]


def test_token_granular_vertical_slash():
    """Token mode: block mask = slash blocks + floor; every selected column is
    attended by every later query (token-level brute force), and the result
    equals the block mode's whenever the columns' blocks are in the mask."""
    rng = np.random.default_rng(31)
    bs, N, d = 8, 61, 16
    q = rng.standard_normal((N, d)).astype(F32)
    k = rng.standard_normal((N, d)).astype(F32)
    v = rng.standard_normal((N, d)).astype(F32)
    k[[3, 20]] += 4.0                                   # two sink columns
    P = O.plan_head(q, k, bs, 0.7, 0.0, bs, vs_granularity=O.VS_TOKEN)
    B = O.plan_head(q, k, bs, 0.7, 0.0, bs)
    assert P.pattern == O.VERTICAL_SLASH and P.cols is not None and P.cols.any()
    assert np.array_equal(P.cols, B.sel_v) and B.cols is None
    nb = -(-N // bs)
    slash = O.apply_floor(O.vs_block_mask(np.zeros(N, bool), P.sel_s, bs), bs, bs)
    assert np.array_equal(P.mask, slash)
    assert not (P.mask & ~B.mask).any()               # never more blocks than block mode
    # token-level definition
    out = O.attend_head(q, k, v, P.mask, bs, P.cols)
    ref = np.zeros((N, d))
    for i in range(N):
        keys = [j for j in range(i + 1) if P.mask[i // bs, j // bs] or P.cols[j]]
        s = np.array([float(q[i].astype(np.float64) @ k[j].astype(np.float64)) for j in keys]) / math.sqrt(d)
        w = np.exp(s - s.max())
        ref[i] = (w / w.sum()) @ v[keys].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # marking every column of the block mode's column blocks reproduces block mode
    colblk = np.zeros(N, bool)
    for kb in np.unique(np.nonzero(B.sel_v)[0] // bs):
        colblk[kb * bs: (kb + 1) * bs] = True
    np.testing.assert_allclose(O.attend_head(q, k, v, P.mask, bs, colblk),
                               O.attend_head(q, k, v, B.mask, bs), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        O.plan_head(q, k, bs, 0.7, 0.0, bs, vs_granularity="lines")
