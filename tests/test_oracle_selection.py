"""Pins of the oracle's cumulative-attention selection, block conversion and
minimum-budget floor: brute force over all subsets, token-level masks and
invariants (no GPU)."""
import itertools

import numpy as np
import pytest

import oracle as O

F32 = np.float32


def _fixed(values, gamma):
    u = [int(round(float(x) * 2 ** 32)) for x in values]
    U = sum(u)
    G = int(round(float(F32(gamma)) * 2 ** 24))
    T = -(-G * U // 2 ** 24)
    return u, T


def brute_force_select(values, gamma):
    """All subsets: the minimal-cardinality subsets whose fixed-point mass
    reaches T; among them the one whose (value desc, index asc) key sequence
    is lexicographically first."""
    n = len(values)
    u, T = _fixed(values, gamma)
    if T == 0:
        return set()
    for size in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            if sum(u[i] for i in sub) >= T:
                key = sorted((-float(values[i]), i) for i in sub)
                if best is None or key < best[0]:
                    best = (key, set(sub))
        if best is not None:
            return best[1]
    raise AssertionError("threshold unreachable")


@pytest.mark.parametrize("seed", range(60))
def test_selection_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 12))
    if seed % 3 == 0:    # many exact ties
        vals = rng.choice(np.array([0.0, 0.125, 0.25, 0.5], F32), size=n)
        if vals.sum() == 0:
            vals[0] = F32(0.5)
    else:
        vals = rng.dirichlet(np.ones(n)).astype(F32)
    gamma = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.999, rng.uniform(0.01, 1.0)]))
    sel = O.select_cumulative(vals, gamma)
    assert set(np.nonzero(sel)[0].tolist()) == brute_force_select(vals, gamma)


def test_selection_invariants_and_monotone_in_gamma():
    rng = np.random.default_rng(11)
    vals = (rng.pareto(1.2, 5000) + 1e-3).astype(F32)
    vals /= vals.sum()
    prev = None
    for gamma in (0.5, 0.8, 0.9, 0.95, 0.99):
        sel = O.select_cumulative(vals, gamma)
        u, T = _fixed(vals, gamma)
        u = np.array(u, dtype=object)
        chosen = np.nonzero(sel)[0]
        mass = sum(u[chosen])
        assert mass >= T
        # dropping the smallest chosen element falls below the threshold
        smallest = min(chosen, key=lambda i: (float(vals[i]), -i))
        assert mass - u[smallest] < T
        # every chosen value >= every unchosen value
        assert vals[sel].min() >= vals[~sel].max()
        # float64 mass reaches gamma up to the fixed-point resolution
        assert vals[sel].astype(np.float64).sum() >= gamma * vals.astype(np.float64).sum() - 1e-6
        if prev is not None:
            assert np.all(sel[prev])                 # S(g1) subset of S(g2)
        prev = sel


def test_selection_ties_prefer_lower_index():
    vals = np.full(10, 0.1, F32)
    sel = O.select_cumulative(vals, 0.35)
    assert np.nonzero(sel)[0].tolist() == [0, 1, 2, 3]


def test_gamma_one_selects_every_nonzero_entry():
    vals = np.array([0.5, 0.0, 0.25, 0.25], F32)
    assert O.select_cumulative(vals, 1.0).tolist() == [True, False, True, True]


def token_level_vs_blocks(sel_cols, sel_diags, bs):
    N = len(sel_cols)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    tok = (j <= i) & (sel_cols[j] | sel_diags[np.clip(i - j, 0, N - 1)])
    nb = -(-N // bs)
    tok = np.pad(tok, ((0, nb * bs - N), (0, nb * bs - N)))
    return tok.reshape(nb, bs, nb, bs).any(axis=(1, 3))


@pytest.mark.parametrize("seed", range(25))
def test_vs_block_mask_equals_token_level_any(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([4, 8, 16]))
    nb = int(rng.integers(1, 10))
    N = bs * nb
    sel_cols = rng.random(N) < rng.uniform(0, 0.2)
    sel_diags = rng.random(N) < rng.uniform(0, 0.2)
    if seed == 0:
        sel_diags[:] = False
        sel_diags[bs] = True           # r = 0: exactly one block diagonal
    got = O.vs_block_mask(sel_cols, sel_diags, bs)
    assert np.array_equal(got, token_level_vs_blocks(sel_cols, sel_diags, bs))


@pytest.mark.parametrize("seed", range(40))
def test_vs_block_mask_ragged_equals_token_level_any(seed):
    """A partial last query block: an offset reaches its own block diagonal
    there only if its remainder is below the block's row count."""
    rng = np.random.default_rng(500 + seed)
    bs = int(rng.choice([4, 8, 16]))
    N = int(rng.integers(1, 10 * bs))
    sel_cols = rng.random(N) < rng.uniform(0, 0.15)
    sel_diags = rng.random(N) < rng.uniform(0, 0.3)
    got = O.vs_block_mask(sel_cols, sel_diags, bs)
    assert np.array_equal(got, token_level_vs_blocks(sel_cols, sel_diags, bs)), (N, bs)


def test_floor_tops_up_nearest_first():
    nb, bs = 12, 16
    mask = np.zeros((nb, nb), bool)
    mask[7, 0] = True
    mask[9, [0, 2, 5, 9]] = True
    out = O.apply_floor(mask, min_budget=3 * bs, bs=bs)
    for qb in range(nb):
        assert out[qb, : qb + 1].sum() >= min(qb + 1, 3)
        assert not out[qb, qb + 1:].any()
    assert np.nonzero(out[7])[0].tolist() == [0, 6, 7]
    assert np.nonzero(out[9])[0].tolist() == [0, 2, 5, 9]      # already >= 3: unchanged
    assert np.nonzero(out[1])[0].tolist() == [0, 1]
    # min_budget 0 still keeps one block per row
    out0 = O.apply_floor(np.zeros((nb, nb), bool), 0, bs)
    assert np.array_equal(out0, np.eye(nb, dtype=bool))
    # a budget that is not a multiple of the block rounds up
    assert O.floor_blocks(1000, 128) == 8 and O.floor_blocks(1024, 128) == 8
    assert O.floor_blocks(2048, 64) == 32 and O.floor_blocks(1, 64) == 1


def test_qa_mask_maps_flattened_triangle():
    nb = 6
    sel = np.zeros(nb * (nb + 1) // 2, bool)
    sel[0] = True           # (0, 0)
    sel[4] = True           # (2, 1): 2*3/2 + 1
    sel[20] = True          # (5, 5)
    m = O.qa_block_mask(sel, nb)
    assert sorted(zip(*np.nonzero(m))) == [(0, 0), (2, 1), (5, 5)]
    A = np.arange(nb * nb, dtype=F32).reshape(nb, nb)
    assert O.tri_values(A)[4] == A[2, 1]


def brute_force_cap(had, scores_row, cap):
    """The cap-subset of a row's blocks chosen by enumeration: every subset of
    ``cap`` blocks is scored by its exact score sum (float32 values summed as
    rationals), and among the subsets with the largest sum the one holding the
    blocks nearest the diagonal wins, i.e. the largest sum of 2^kb (two such
    subsets differ first in their largest differing block).  Nothing here
    sorts by the oracle's (score, block) key."""
    from fractions import Fraction
    best, best_key = None, None
    for sub in itertools.combinations(had, cap):
        key = (sum(Fraction(float(scores_row[kb])) for kb in sub), sum(1 << int(kb) for kb in sub))
        if best_key is None or key > best_key:
            best, best_key = set(int(x) for x in sub), key
    return best


@pytest.mark.parametrize("seed", range(20))
def test_cap_keeps_highest_scoring_blocks(seed):
    rng = np.random.default_rng(300 + seed)
    nb, bs = int(rng.integers(1, 14)), 16
    mask = np.tril(rng.random((nb, nb)) < rng.uniform(0.2, 1.0))
    mask = O.apply_floor(mask, bs, bs)
    # odd seeds: few distinct scores, so many rows are decided by the tie rule
    scores = rng.choice(np.array([0.0, 0.25, 0.5, 1.0], np.float32), size=(nb, nb)) if seed % 2 \
        else rng.random((nb, nb)).astype(np.float32)
    cap = int(rng.integers(1, 6))
    out = O.apply_cap(mask, scores, cap * bs, bs)
    assert np.array_equal(O.apply_cap(mask, scores, 0, bs), mask)
    for qb in range(nb):
        kept = set(np.nonzero(out[qb])[0].tolist())
        had = np.nonzero(mask[qb])[0].tolist()
        if len(had) <= cap:
            assert kept == set(had)
            continue
        assert kept == brute_force_cap(had, scores[qb], cap), (qb, had, scores[qb, had].tolist(), cap)
    assert O.cap_blocks(8192, 128) == 64 and O.cap_blocks(1, 64) == 1 and O.cap_blocks(0, 64) == 0


def test_cap_tie_rule_hand_case():
    """Worked by hand: blocks 0..4 of row 4 with scores 0.5, 0.9, 0.5, 0.1,
    0.5 and a cap of 3 blocks keep 1 (the largest score) and, of the three
    blocks tied at 0.5, the two nearest the diagonal (4 and 2)."""
    mask = np.tril(np.ones((5, 5), bool))
    scores = np.zeros((5, 5), np.float32)
    scores[4] = [0.5, 0.9, 0.5, 0.1, 0.5]
    out = O.apply_cap(mask, scores, 3 * 32, 32)
    assert np.nonzero(out[4])[0].tolist() == [1, 2, 4]
    assert np.nonzero(out[2])[0].tolist() == [0, 1, 2]   # rows within the cap are unchanged


@pytest.mark.parametrize("seed", range(10))
def test_vs_block_scores_equal_touching_line_mass(seed):
    """score(qb, kb) = mass of the selected lines that touch block (qb, kb),
    enumerated at token level (a column j or an offset o touches the block iff
    some causal (i, j) in it has that column or that offset)."""
    rng = np.random.default_rng(400 + seed)
    bs, nb = 8, int(rng.integers(1, 7))
    N = bs * nb
    c = rng.random(N).astype(np.float32)
    g = rng.random(N).astype(np.float32)
    sel_c = rng.random(N) < 0.3
    sel_g = rng.random(N) < 0.3
    got = O.vs_block_scores(c, g, sel_c, sel_g, bs)
    for qb in range(nb):
        for kb in range(qb + 1):
            i = qb * bs + np.arange(bs)[:, None]
            j = kb * bs + np.arange(bs)[None, :]
            i, j = np.broadcast_arrays(i, j)
            causal = j <= i
            cols = {int(x) for x in j[causal].ravel()}
            offs = {int(x) for x in (i - j)[causal].ravel()}
            ref = sum(float(c[x]) for x in cols if sel_c[x]) + sum(float(g[x]) for x in offs if sel_g[x])
            assert abs(float(got[qb, kb]) - ref) <= 1e-5 * max(1.0, ref)


def test_querywise_selection_rows():
    """Each row of the query-wise mask is the brute-force minimal set of its
    own estimated row; gamma = 1 keeps every nonzero entry."""
    rng = np.random.default_rng(77)
    nb = 7
    A = np.zeros((nb, nb), F32)
    for qb in range(nb):
        row = rng.dirichlet(np.ones(qb + 1) * 0.5).astype(F32)
        if qb == 3:
            row[:] = F32(0.25)             # exact ties: lower key blocks first
        A[qb, : qb + 1] = row
    for gamma in (0.3, 0.7, 0.95):
        m = O.qa_querywise_mask(A, gamma)
        assert not np.triu(m, 1).any()
        for qb in range(nb):
            assert set(np.nonzero(m[qb])[0].tolist()) == brute_force_select(A[qb, : qb + 1], gamma)
    assert np.nonzero(O.qa_querywise_mask(A, 0.5)[3])[0].tolist() == [0, 1]


def test_querywise_plan_differs_only_for_query_aware_heads():
    from synth import BY_NAME, LayerGen
    cfg = BY_NAME["tiny_fp32_4k"].with_(N=2048)
    q, k, _ = LayerGen(cfg).numpy_layer()
    seen = set()
    for h in range(cfg.Hq):
        a = O.plan_head(q[0, h], k[0, h], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget)
        b = O.plan_head(q[0, h], k[0, h], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget,
                        qa_selection=O.QA_QUERYWISE)
        assert a.pattern == b.pattern and a.D == b.D
        seen.add(a.pattern)
        if a.pattern == O.VERTICAL_SLASH:
            assert np.array_equal(a.mask, b.mask)
        else:
            # every row reaches gamma of its own estimated mass (before the floor)
            sel = O.qa_querywise_mask(a.A, cfg.gamma)
            for qb in range(cfg.nb):
                row = a.A[qb, : qb + 1].astype(np.float64)
                assert row[sel[qb, : qb + 1]].sum() >= cfg.gamma * row.sum() - 1e-6
            assert np.array_equal(b.mask, O.apply_floor(sel, cfg.min_budget, cfg.block))
    assert seen == {O.QUERY_AWARE, O.VERTICAL_SLASH}
    with pytest.raises(ValueError):
        O.plan_head(q[0, 0], k[0, 0], cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, qa_selection="rows")
