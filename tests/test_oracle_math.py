"""Pins of the oracle's canonical arithmetic against libm, library routines
and closed forms (no GPU)."""
import math

import numpy as np
import pytest
import scipy.spatial.distance as ssd
import scipy.special
import torch

import oracle as O

F32, F64 = np.float32, np.float64


def ulp_err32(y, ref):
    ref32 = ref.astype(F32)
    sp = np.spacing(np.abs(ref32)).astype(F64)
    return np.max(np.abs(y.astype(F64) - ref) / sp)


def test_exp2_matches_libm_within_2ulp():
    x = np.concatenate([np.linspace(-100, 0, 1_000_001, dtype=F32),
                        np.maximum(-np.abs(np.random.default_rng(1).standard_normal(100_000).astype(F32)) * 30, F32(-100))])
    y = O.exp2_c(x)
    assert ulp_err32(y, np.exp2(x.astype(F64))) <= 2.0


def test_exp2_special_points():
    assert O.exp2_c(np.array([0.0], F32))[0] == F32(1.0)
    ints = -np.arange(0, 101, dtype=F32)
    assert np.array_equal(O.exp2_c(ints), np.ldexp(F32(1.0), (-np.arange(0, 101)).astype(np.int32)).astype(F32))
    assert O.exp2_c(np.array([-100.5, -1e30, -np.inf], F32)).tolist() == [0.0, 0.0, 0.0]
    assert O.exp2_c(np.array([-100.0], F32))[0] == F32(2.0 ** -100)


def test_exp2_coefficients_are_taylor_terms_of_2_pow_f():
    # c0 = 1 and c1 = ln 2 rounded to fp32 (libm's value), c_k ~ (ln 2)^k / k!
    assert O.EXP2_COEF[0] == F32(1.0)
    assert O.EXP2_COEF[1] == F32(math.log(2.0))
    for k, c in enumerate(O.EXP2_COEF):
        assert abs(float(c) - math.log(2.0) ** k / math.factorial(k)) <= 2 ** -24 * float(c)


def test_ln_matches_libm():
    rng = np.random.default_rng(2)
    x = np.exp(rng.uniform(-700, 700, 200_000))
    x = np.concatenate([x, np.linspace(0.5, 2.0, 100_001), [1e-300, 1e300, 5e-324 * 2 ** 60]])
    y = O.ln_c(x)
    ref = np.log(x)
    err = np.abs(y - ref) / np.maximum(np.spacing(np.abs(ref)), np.spacing(1.0) * 0.5)
    assert err.max() <= 4.0


def test_ln_exact_points():
    assert O.ln_c(np.array([1.0]))[0] == 0.0
    assert O.ln_c(np.array([2.0]))[0] == F64(math.log(2.0))
    assert O.ln_c(np.array([0.5]))[0] == -F64(math.log(2.0))
    assert O.LN2_F64 == F64(math.log(2.0))


def test_score_scale_is_log2e_over_sqrt_d():
    for d in (64, 128, 256):
        C = O.score_scale(d)
        assert abs(float(C) - math.log2(math.e) / math.sqrt(d)) <= 2 ** -24 * float(C)
        assert C.dtype == F32


def test_dot_seq_close_to_float64_and_equals_fused_for_bf16_inputs():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((7, 128)).astype(F32)
    b = rng.standard_normal((33, 128)).astype(F32)
    s = O.dot_seq(a, b)
    ref = a.astype(F64) @ b.astype(F64).T
    bound = 128 * 2 ** -23 * (np.abs(a).astype(F64) @ np.abs(b).astype(F64).T)
    assert np.all(np.abs(s - ref) <= bound)
    # For bf16-representable inputs every product is exact in fp32, so the
    # separately rounded product-then-add equals one fused multiply-add.
    ab = torch.from_numpy(a).bfloat16().float().numpy()
    bb = torch.from_numpy(b).bfloat16().float().numpy()
    s = O.dot_seq(ab, bb)
    acc = np.zeros((7, 33), F32)
    for t in range(128):
        acc = (acc.astype(F64) + ab[:, t:t + 1].astype(F64) * bb[None, :, t].astype(F64)).astype(F32)
    assert np.array_equal(s, acc)
    # the reduction is sequential in t: reversing t changes the rounding
    s_rev = O.dot_seq(a[:, ::-1], b[:, ::-1])
    assert not np.array_equal(s_rev, O.dot_seq(a, b))


def test_pool_mean_matches_avg_pool():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1024, 128)).astype(F32)
    for bs in (64, 128):
        p = O.pool_mean(x, bs)
        ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x).double().T[None], bs, bs)[0].T.numpy()
        np.testing.assert_allclose(p, ref, rtol=0, atol=1e-6)


def test_pool_mean_ragged_tail_is_the_mean_of_the_rows_present():
    rng = np.random.default_rng(41)
    for n, bs in ((1000, 128), (64 * 3 + 1, 64), (37, 64)):
        x = rng.standard_normal((n, 128)).astype(F32)
        p = O.pool_mean(x, bs)
        nb = -(-n // bs)
        assert p.shape == (nb, 128)
        for kb in range(nb):
            ref = x[kb * bs: (kb + 1) * bs].astype(F64).mean(axis=0)
            np.testing.assert_allclose(p[kb], ref, rtol=0, atol=2e-6)
        # full blocks: identical to the exact 1/bs scaling
        full = n // bs
        if full:
            acc = np.zeros((full, 128), F32)
            for r in range(bs):
                acc = acc + x[: full * bs].reshape(full, bs, 128)[:, r]
            assert np.array_equal(p[:full], acc * F32(1.0 / bs))


def _ideal_last_block(q, k, bs):
    """float64 causal softmax of the last min(bs, N) queries, via torch
    library calls."""
    N, d = q.shape
    R = min(bs, N)
    qt = torch.from_numpy(q).double()[N - R:]
    kt = torch.from_numpy(k).double()
    s = qt @ kt.T / math.sqrt(d)
    pos = torch.arange(N - R, N)[:, None]
    s = s.masked_fill(torch.arange(N)[None, :] > pos, float("-inf"))
    p = torch.softmax(s, dim=1)
    c = p.sum(0)
    # diagonal sums: g[o] = sum_i p[i, pos_i - o] -> put p in an N x N causal frame
    full = torch.zeros(N, N, dtype=torch.float64)
    full[N - R:] = p
    g = torch.stack([torch.diagonal(full, offset=-o).sum() for o in range(N)])
    nb = -(-N // bs)
    a = torch.nn.functional.pad(c, (0, nb * bs - N)).reshape(nb, bs).sum(1)
    return p.numpy(), c.numpy(), g.numpy(), (a / a.sum()).numpy()


@pytest.mark.parametrize("bs", [64, 128])
def test_last_block_stats_match_float64_softmax(bs):
    rng = np.random.default_rng(5 + bs)
    N, d = 8 * bs, 128
    q = rng.standard_normal((N, d)).astype(F32)
    k = rng.standard_normal((N, d)).astype(F32)
    k[5] += 3.0                     # a mild sink so the mass is uneven
    st = O.last_block_stats(q, k, bs)
    p, c, g, a = _ideal_last_block(q, k, bs)
    np.testing.assert_allclose(st.c, c, rtol=2e-5, atol=1e-8)
    np.testing.assert_allclose(st.g, g, rtol=2e-5, atol=1e-8)
    np.testing.assert_allclose(st.a_true, a, rtol=2e-5, atol=1e-9)
    # c and g each sum to the number of query rows (every row is a distribution)
    assert abs(float(st.c.astype(F64).sum()) - bs) < 1e-3
    assert abs(float(st.g.astype(F64).sum()) - bs) < 1e-3
    # causality: the last query row sees the whole sequence, the first only N-bs+1 keys
    assert st.g[N - bs + 1:].max() <= c.max()


@pytest.mark.parametrize("N,bs", [(1000, 128), (8 * 64 + 5, 64), (100, 128), (1, 64)])
def test_last_block_stats_ragged(N, bs):
    """N not a multiple of the block (and N below one block): the last
    min(bs, N) queries, a partial last key block."""
    rng = np.random.default_rng(N)
    q = rng.standard_normal((N, 128)).astype(F32)
    k = rng.standard_normal((N, 128)).astype(F32)
    st = O.last_block_stats(q, k, bs)
    p, c, g, a = _ideal_last_block(q, k, bs)
    R = min(bs, N)
    assert st.M.shape == (R,) and st.a_true.shape == (-(-N // bs),)
    np.testing.assert_allclose(st.c, c, rtol=2e-5, atol=1e-8)
    np.testing.assert_allclose(st.g, g, rtol=2e-5, atol=1e-8)
    np.testing.assert_allclose(st.a_true, a, rtol=2e-5, atol=1e-9)
    assert abs(float(st.c.astype(F64).sum()) - R) < 1e-3


def test_estimate_map_matches_float64_softmax():
    rng = np.random.default_rng(6)
    nb, d = 40, 128
    qb = rng.standard_normal((nb, d)).astype(F32) * 3
    kb = rng.standard_normal((nb, d)).astype(F32) * 3
    A = O.estimate_map(qb, kb)
    s = torch.from_numpy(qb).double() @ torch.from_numpy(kb).double().T / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(nb, nb, dtype=torch.bool), 1), float("-inf"))
    ref = torch.softmax(s, 1).numpy()
    np.testing.assert_allclose(A, ref, rtol=2e-5, atol=1e-9)
    assert np.all(np.triu(A, 1) == 0)
    assert A[0, 0] == F32(1.0)


def test_jsd_identities():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(2, 300))
        p = rng.dirichlet(np.ones(n) * rng.uniform(0.05, 3)).astype(F32)
        q = rng.dirichlet(np.ones(n) * rng.uniform(0.05, 3)).astype(F32)
        j0, d0 = O.jsd_canonical(p, p)
        assert j0 == 0.0 and d0 == 0.0
        j1, d1 = O.jsd_canonical(p, q)
        j2, d2 = O.jsd_canonical(q, p)
        assert j1 == j2 and d1 == d2                  # exactly symmetric
        assert 0.0 <= d1 <= math.sqrt(math.log(2.0))
        P, Q = p.astype(F64), q.astype(F64)
        M = 0.5 * (P + Q)
        ref_j = 0.5 * (scipy.special.rel_entr(P, M).sum() + scipy.special.rel_entr(Q, M).sum())
        assert abs(j1 - ref_j) <= 1e-15 + 1e-12 * ref_j
        # scipy's distance renormalises its inputs (fp32 sums differ from 1 by ~1e-7)
        ref = ssd.jensenshannon(P, Q)              # natural base
        assert abs(d1 - ref) <= 1e-6


def test_jsd_disjoint_supports_is_ln2():
    p = np.array([1.0, 0.0, 0.0, 0.0], F32)
    q = np.array([0.0, 0.5, 0.25, 0.25], F32)
    j, d = O.jsd_canonical(p, q)
    assert j == math.log(2.0)
    assert d == math.sqrt(math.log(2.0))


@pytest.mark.parametrize("a,b", [(0.3, 0.6), (0.01, 0.99), (0.5, 0.5), (0.0, 0.25)])
def test_jsd_two_point_closed_form(a, b):
    p = np.array([a, 1 - a], F32)
    q = np.array([b, 1 - b], F32)
    P, Q = p.astype(F64), q.astype(F64)

    def h(x):
        return -sum(t * math.log(t) for t in x if t > 0)
    ref = h((P + Q) / 2) - 0.5 * (h(P) + h(Q))
    j, _ = O.jsd_canonical(p, q)
    assert abs(j - ref) <= 1e-15 + 1e-12 * abs(ref)


def test_divergence_closed_form_with_block_constant_keys():
    """Keys constant inside each block and identical last-block queries: the
    pooled estimate sees the block scores exactly, the true distribution
    differs only through the causal truncation inside the diagonal block."""
    rng = np.random.default_rng(8)
    bs, nb, d = 64, 12, 128
    N = bs * nb
    kv = (rng.integers(-4, 5, size=(nb, d)) / 8.0).astype(F32)
    k = np.repeat(kv, bs, axis=0)
    qv = (rng.integers(-4, 5, size=d) / 8.0).astype(F32)
    q = rng.standard_normal((N, d)).astype(F32)
    q[N - bs:] = qv                        # all last-block queries identical
    q[(nb - 1) * bs:] = qv
    P = O.plan_head(q, k, bs, 0.95, 0.1, 0)
    s = (kv.astype(F64) @ qv.astype(F64)) / math.sqrt(d)
    est = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    # true: query i of the last block sees all keys of blocks < nb-1 and i+1
    # keys of the last block
    tru = np.zeros(nb)
    for i in range(bs):
        w = np.exp(s - s.max()) * bs
        w[-1] = np.exp(s[-1] - s.max()) * (i + 1)
        tru += w / w.sum()
    tru /= tru.sum()
    np.testing.assert_allclose(P.A[nb - 1], est, rtol=1e-5, atol=1e-12)
    np.testing.assert_allclose(P.stats.a_true, tru, rtol=1e-5, atol=1e-12)
    m = (est + tru) / 2
    jsd = 0.5 * (np.sum(est * np.log(est / m)) + np.sum(tru * np.log(tru / m)))
    assert abs(P.D - math.sqrt(jsd)) <= 1e-6
