"""Property-based pins of the oracle's selection and block conversion (no GPU).

Inputs are drawn by hypothesis, derandomised so that every run checks the
same cases: unnormalised float32 masses with exact zeros, ties, subnormals and
values far apart in magnitude, any gamma in (0, 1], and random vertical /
slash line selections at ragged lengths.  Each case is compared with a
definition written out independently: the subset brute force of the
cumulative selection, and the block mask obtained by marking every causal
(query, key) pair a selected line covers.
"""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle as O  # noqa: E402
from tests.test_oracle_selection import brute_force_select  # noqa: E402

F32 = np.float32
SETTINGS = settings(derandomize=True, max_examples=400, deadline=None, database=None)

# float32 masses: exact zeros, subnormals, dyadic values (exact ties) and
# arbitrary values over several orders of magnitude
_mass = st.one_of(
    st.just(0.0),
    st.sampled_from([1e-45, 1e-40, 2.0 ** -20, 0.125, 0.25, 0.5, 1.0]),
    st.floats(min_value=float(F32(1e-6)), max_value=1.0, allow_nan=False, allow_infinity=False, width=32),
)
_gamma = st.one_of(st.sampled_from([1.0, 0.95, 0.9, 0.5]),
                   st.floats(min_value=float(F32(1e-3)), max_value=1.0, allow_nan=False, width=32))


@SETTINGS
@given(vals=st.lists(_mass, min_size=1, max_size=9), gamma=_gamma)
def test_selection_is_the_subset_brute_force(vals, gamma):
    v = np.array(vals, F32)
    sel = O.select_cumulative(v, gamma)
    assert set(np.nonzero(sel)[0].tolist()) == brute_force_select(v, gamma)


@SETTINGS
@given(vals=st.lists(_mass, min_size=1, max_size=40), gamma=_gamma)
def test_selection_reaches_gamma_and_is_a_prefix_of_the_order(vals, gamma):
    v = np.array(vals, F32)
    sel = O.select_cumulative(v, gamma)
    u = np.array([int(round(float(x) * 2 ** 32)) for x in v], dtype=object)
    U = int(u.sum())
    G = int(round(float(F32(gamma)) * 2 ** 24))
    T = -(-G * U // 2 ** 24)
    got = int(u[sel].sum()) if sel.any() else 0
    assert got >= T
    # the selected entries come first in (value descending, index ascending) order
    order = sorted(range(len(v)), key=lambda i: (-float(v[i]), i))
    k = int(sel.sum())
    assert set(order[:k]) == set(np.nonzero(sel)[0].tolist())
    # and the prefix one entry shorter does not reach the threshold
    if k:
        assert int(sum(u[i] for i in order[: k - 1])) < T


@st.composite
def _lines(draw):
    bs = draw(st.sampled_from([2, 3, 4, 8]))
    N = draw(st.integers(min_value=1, max_value=6 * bs))
    cols = np.array(draw(st.lists(st.booleans(), min_size=N, max_size=N)), bool)
    diags = np.array(draw(st.lists(st.booleans(), min_size=N, max_size=N)), bool)
    return cols, diags, bs


@SETTINGS
@given(case=_lines())
def test_block_conversion_is_the_token_level_cover(case):
    cols, diags, bs = case
    N = cols.size
    nb = -(-N // bs)
    want = np.zeros((nb, nb), bool)
    for i in range(N):
        for j in range(i + 1):
            if cols[j] or diags[i - j]:
                want[i // bs, j // bs] = True
    np.testing.assert_array_equal(O.vs_block_mask(cols, diags, bs), want)


@st.composite
def _masks(draw):
    nb = draw(st.integers(min_value=1, max_value=12))
    bs = draw(st.sampled_from([64, 128]))
    bits = draw(st.lists(st.booleans(), min_size=nb * nb, max_size=nb * nb))
    mask = np.tril(np.array(bits, bool).reshape(nb, nb))
    min_budget = draw(st.integers(min_value=0, max_value=14 * bs))
    return mask, bs, min_budget


@SETTINGS
@given(case=_masks())
def test_floor_adds_the_nearest_missing_blocks(case):
    mask, bs, min_budget = case
    nb = mask.shape[0]
    out = O.apply_floor(mask, min_budget, bs)
    f = max(1, -(-min_budget // bs))
    for qb in range(nb):
        want = mask[qb].copy()
        need = min(qb + 1, f) - int(want.sum())
        for kb in range(qb, -1, -1):          # nearest the diagonal first
            if need <= 0:
                break
            if not want[kb]:
                want[kb] = True
                need -= 1
        np.testing.assert_array_equal(out[qb], want, err_msg=f"row {qb}")
    assert not np.triu(out, 1).any()
