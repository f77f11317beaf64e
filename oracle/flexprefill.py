"""CPU oracle for FlexPrefill sparse pre-filling attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant
table or helper with the HIP library; it is written from the FlexPrefill
pages and is deliberately plain and slow.

What FlexPrefill computes (FlexPrefill, ICLR 2025 submission 1022; abstract
on the OpenReview and codewithpapers pages, "Approach" paragraph of the
atlas.scime.ai summary page):

1. Query-aware sparse pattern determination: for every attention head the
   attention of the last query block over all keys (the "true
   distribution"), pooled per key block, is compared with an estimate built
   from block-pooled queries and keys using the square root of the
   Jensen-Shannon divergence.  If the estimate is accurate (divergence below
   tau) the head uses the query-aware pattern, otherwise the vertical-slash
   pattern.
2. Cumulative-attention index selection: the smallest set of blocks (query-
   aware) or lines (vertical key columns and slash diagonals) whose summed
   normalised attention reaches gamma; the ablation table adds a minimum
   budget (1024 tokens by default) and selects over the flattened estimated
   map rather than row by row.
3. Sparse attention restricted to the selected blocks.

The pages give no formulas, so the oracle fixes one exact arithmetic for
the selection half (``canonical``: every float32 / float64 rounding point
and reduction order spelled out, the gamma test done on integers) so that
an independent GPU implementation can reproduce pattern choices and block
lists bit for bit.  The attention half is the plain definition in float64.

Readings of points the pages leave open (each is listed with its reason in
the design notes of the repository):
  * softmax scale 1/sqrt(d), folded with log2(e) into one fp32 constant;
  * representative queries = the last ``block`` queries, attending causally;
  * pooling = block mean; the estimate includes the diagonal block;
  * divergence uses natural logarithms, D = sqrt(JSD) in [0, sqrt(ln 2)];
  * query-aware iff D < tau (strict, so tau = 0 disables it);
  * "reaches gamma" = selected mass >= gamma * total, in fixed point;
  * ties broken by value descending, then index ascending;
  * vertical and slash lines are selected separately, each to gamma of its
    own total, and turned into blocks by the any-touch rule;
  * minimum budget = ceil(min_budget / block) blocks per query-block row
    (at least 1), filled nearest-first from the diagonal;
  * gamma = 1 selects the whole causal triangle;
  * an optional maximum budget caps every query-block row at
    ceil(max_budget / block) blocks, keeping the blocks with the largest
    estimate (query-aware) or selected line mass (vertical-slash), ties
    to the block nearest the diagonal;
  * the optional query-wise selection applies the same cumulative rule to
    each estimated row on its own instead of to the flattened map;
  * the optional token-granular vertical-slash mode attends a vertical-slash
    head's selected columns token by token and keeps only its slash blocks
    and the minimum-budget fill (and cap) as whole blocks.

Pins (tests in ``tests/test_oracle_*.py``): exp2_c / ln_c against libm
within a few ulp; JSD against scipy and closed forms; canonical softmax
statistics, pooling and the estimate against float64 library computations;
selection against brute force over all subsets; the block conversion
against a token-level mask; attention against torch's scaled-dot-product
attention (gamma = 1) and a per-token brute force; hand-worked selections,
line-to-block conversions and divergences stored under ``tests/golden/``.
Parity unpinned: that
the conventions above are the authors' own rules -- the pages print no
formulas, listings or intermediate values to check them against.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, Iterable, List, Optional

import numpy as np

F32 = np.float32
F64 = np.float64

# --------------------------------------------------------------------------
# Canonical arithmetic primitives.
# --------------------------------------------------------------------------


def _nearest_f32(x: Fraction) -> np.float32:
    """float32 nearest to the exact rational ``x`` (round half to even).

    float(Fraction) is correctly rounded to binary64; the binary64 value is
    then rounded to binary32.  The double rounding can only differ from a
    direct rounding when the binary64 value sits exactly on a binary32
    midpoint, which is checked and refused."""
    d = float(x)
    f = np.float32(d)
    lo = np.nextafter(f, F32(-np.inf)) if f > 0 else f
    hi = np.nextafter(f, F32(np.inf))
    for nb_ in (lo, hi):
        mid = (Fraction(float(f)) + Fraction(float(nb_))) / 2
        if Fraction(d) == mid:
            raise ArithmeticError("double rounding ambiguity")
    return f


def _ln2_fraction(digits: int = 60) -> Fraction:
    """ln 2 as a rational accurate to ~``digits`` decimal digits, from the
    series ln 2 = sum_{k>=1} 1 / (k 2^k)."""
    acc = Fraction(0)
    k = 1
    while True:
        term = Fraction(1, k * 2 ** k)
        acc += term
        if term < Fraction(1, 10 ** digits):
            return acc
        k += 1


_LN2_Q = _ln2_fraction()
# Taylor coefficients of 2^f = exp(f ln 2): c_k = (ln 2)^k / k!, nearest fp32.
EXP2_COEF = tuple(_nearest_f32(_LN2_Q ** k / math.factorial(k)) for k in range(8))
# artanh series: ln m = 2 artanh z = 2 z sum_k z^(2k) / (2k + 1), fp64 nearest.
LN_COEF = tuple(F64(1.0) / F64(2 * k + 1) for k in range(11))
LN2_F64 = F64(float(_LN2_Q))
SQRT_HALF_F64 = np.sqrt(F64(0.5))


def exp2_c(x: np.ndarray) -> np.ndarray:
    """2^x for float32 x <= 0 in canonical float32 arithmetic.

    x < -100 gives +0.  Otherwise n = rint(x), f = x - n (exact, |f| <= 1/2),
    p = Horner evaluation of sum_k c_k f^k for k = 7..0 with every product
    and sum rounded to float32 (no fused multiply-add), result p * 2^n.
    Cody-Waite style integer/fraction split with a degree-7 Taylor series
    (truncation < 6e-9 relative)."""
    x = np.asarray(x, dtype=F32)
    out = np.zeros(x.shape, dtype=F32)
    live = x >= F32(-100.0)
    xs = x[live]
    n = np.rint(xs)
    f = xs - n
    p = np.full(xs.shape, EXP2_COEF[7], dtype=F32)
    for k in range(6, -1, -1):
        p = p * f
        p = p + EXP2_COEF[k]
    out[live] = np.ldexp(p, n.astype(np.int32)).astype(F32)
    return out


def ln_c(x: np.ndarray) -> np.ndarray:
    """Natural logarithm of float64 x > 0 in canonical float64 arithmetic.

    (m, e) = frexp(x); if m < sqrt(1/2) then m = 2m, e = e - 1; z = (m-1)/(m+1);
    ln x = e ln 2 + 2z * sum_{k=0..10} z^(2k)/(2k+1) (Horner in w = z^2),
    every operation rounded to float64 (the artanh / Gregory series)."""
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    small = m < SQRT_HALF_F64
    m = np.where(small, m * F64(2.0), m)
    e = np.where(small, e - 1, e)
    z = (m - F64(1.0)) / (m + F64(1.0))
    w = z * z
    s = np.full(x.shape, LN_COEF[10], dtype=F64)
    for k in range(9, -1, -1):
        s = s * w
        s = s + LN_COEF[k]
    return e.astype(F64) * LN2_F64 + (F64(2.0) * z) * s


def score_scale(d: int) -> np.float32:
    """C = log2(e) / sqrt(d), computed in float64 and rounded once to float32,
    so that exp2(score * C) = exp(q.k / sqrt(d))."""
    log2e = F64(float(1 / _LN2_Q))      # binary64 nearest to log2(e)
    return F32(log2e / np.sqrt(F64(d)))


def dot_seq(a: np.ndarray, b: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """All dot products of rows of a [m, d] with rows of b [n, d] in float32:
    acc = +0; for t = 0..d-1: acc = acc + a[t] * b[t], the product rounded,
    then the sum rounded.  Returns [m, n]."""
    a = np.ascontiguousarray(a, dtype=F32)
    bt = np.ascontiguousarray(np.asarray(b, dtype=F32).T)
    m, d = a.shape
    n = bt.shape[1]
    out = np.empty((m, n), dtype=F32)
    for j0 in range(0, n, chunk):
        j1 = min(n, j0 + chunk)
        acc = np.zeros((m, j1 - j0), dtype=F32)
        for t in range(d):
            prod = a[:, t:t + 1] * bt[t:t + 1, j0:j1]
            acc += prod
        out[:, j0:j1] = acc
    return out


def pool_mean(x: np.ndarray, bs: int) -> np.ndarray:
    """Block average ("block-pooled", Approach paragraph): for each block of
    ``bs`` rows (the last block holds the remaining N - (nb-1) bs rows when
    N is not a multiple of bs) the rows are summed in ascending order in
    float32 and the sum is divided by the block's row count (one rounded
    division; for a full block it equals the exact scaling by 1/bs)."""
    x = np.asarray(x, dtype=F32)
    n, d = x.shape
    nb = -(-n // bs)
    out = np.zeros((nb, d), dtype=F32)
    for kb in range(nb):
        rows = x[kb * bs: min(n, kb * bs + bs)]
        acc = np.zeros(d, dtype=F32)
        for r in range(rows.shape[0]):
            acc = acc + rows[r]
        out[kb] = acc / F32(rows.shape[0])
    return out


def seq_sum_rows(x: np.ndarray) -> np.ndarray:
    """Sequential float32 sum along the last axis, ascending index."""
    x = np.asarray(x, dtype=F32)
    acc = np.zeros(x.shape[:-1], dtype=F32)
    for j in range(x.shape[-1]):
        acc = acc + x[..., j]
    return acc


# --------------------------------------------------------------------------
# Step 1: pattern determination (Approach paragraph; abstract item 1).
# --------------------------------------------------------------------------


@dataclass
class LastBlockStats:
    M: np.ndarray        # [bs] row maxima of the scaled scores
    zpart: np.ndarray    # [bs, nb] per key-block sums of exp2_c(s - M)
    Z: np.ndarray        # [bs] row sums
    c: np.ndarray        # [N] column sums of the probabilities (vertical lines)
    g: np.ndarray        # [N] diagonal sums, offset o = i - j (slash lines)
    a_true: np.ndarray   # [nb] block-pooled true distribution


def _pad_blocks(x: np.ndarray, nb: int, bs: int) -> np.ndarray:
    """x [..., N] zero-padded to [..., nb, bs] (padding adds +0 to sums)."""
    pad = nb * bs - x.shape[-1]
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,), dtype=x.dtype)], axis=-1)
    return x.reshape(x.shape[:-1] + (nb, bs))


def last_block_stats(q: np.ndarray, k: np.ndarray, bs: int) -> LastBlockStats:
    """Exact causal softmax attention of the last ``bs`` queries over all keys
    (the "true distribution" of the Approach paragraph), summarised three ways:
    per key column, per diagonal offset and per key block.

    The representative rows are the last R = min(bs, N) queries; row i sits
    at position pos_i = N - R + i and sees keys j <= pos_i.
    s[i, j] = fp32(dot_seq(q_i, k_j)) * C; M_i = max_j s[i, j];
    e = exp2_c(s - M_i) (0 for j > pos_i); zpart[i, kb] = sequential sum over
    the keys of block kb; Z_i = sequential sum of zpart over kb;
    p = e * fp32(1 / Z_i).  c[j] = sum over i ascending of p[i, j];
    g[o] = sum over i ascending with pos_i >= o of p[i, pos_i - o];
    a_true[kb] = t[kb] / T with t[kb] the sequential sum of c over block kb
    and T the sequential sum of t.  A partial last key block simply holds
    fewer keys."""
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    N, d = q.shape
    nb = -(-N // bs)
    R = min(bs, N)
    C = score_scale(d)
    pos = N - R + np.arange(R)
    s = dot_seq(q[N - R:], k) * C
    valid = np.arange(N)[None, :] <= pos[:, None]
    M = np.where(valid, s, F32(-np.inf)).max(axis=1).astype(F32)
    x = np.where(valid, s - M[:, None], F32(-np.inf)).astype(F32)
    e = exp2_c(x)
    zpart = seq_sum_rows(_pad_blocks(e, nb, bs))
    Z = seq_sum_rows(zpart)
    rZ = F32(1.0) / Z
    p = e * rZ[:, None]
    c = np.zeros(N, dtype=F32)
    g = np.zeros(N, dtype=F32)
    for i in range(R):
        c = c + p[i]
        pi = pos[i]
        g[: pi + 1] = g[: pi + 1] + p[i, pi::-1]
    t = seq_sum_rows(_pad_blocks(c, nb, bs))
    T = seq_sum_rows(t[None, :])[0]
    a_true = t / T
    return LastBlockStats(M=M, zpart=zpart, Z=Z, c=c, g=g, a_true=a_true.astype(F32))


def estimate_map(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Estimated block attention map from block-pooled queries and keys:
    A[qb, kb] = softmax over kb <= qb of fp32(dot_seq(qbar_qb, kbar_kb)) * C,
    with the row maximum subtracted, exp2_c, a sequential row sum over kb
    ascending and a rounded division.  Entries above the diagonal are 0."""
    nb, d = qbar.shape
    C = score_scale(d)
    s = dot_seq(qbar, kbar) * C
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    mx = np.where(tri, s, F32(-np.inf)).max(axis=1).astype(F32)
    x = np.where(tri, s - mx[:, None], F32(-np.inf)).astype(F32)
    e = exp2_c(x)
    Zr = seq_sum_rows(e)
    return (e / Zr[:, None]).astype(F32)


def jsd_canonical(p32: np.ndarray, q32: np.ndarray):
    """Jensen-Shannon divergence (natural log) and its square root D.

    P, Q widened to float64; m = 0.5 (P + Q); term = P ln(P/m) + Q ln(Q/m)
    with a term taken as 0 where its probability is 0; JSD = 0.5 * (sequential
    sum of the terms over kb ascending); D = sqrt(max(JSD, 0))."""
    P = np.asarray(p32, dtype=F32).astype(F64)
    Q = np.asarray(q32, dtype=F32).astype(F64)
    m = F64(0.5) * (P + Q)
    with np.errstate(divide="ignore", invalid="ignore"):
        rp = np.where(P > 0, P / np.where(m > 0, m, 1.0), 1.0)
        rq = np.where(Q > 0, Q / np.where(m > 0, m, 1.0), 1.0)
    tP = np.where(P > 0, P * ln_c(rp), F64(0.0))
    tQ = np.where(Q > 0, Q * ln_c(rq), F64(0.0))
    term = tP + tQ
    acc = 0.0
    for x in term:
        acc = acc + float(x)
    jsd = 0.5 * acc
    return jsd, math.sqrt(max(jsd, 0.0))


# --------------------------------------------------------------------------
# Step 2: cumulative-attention index selection (abstract item 2).
# --------------------------------------------------------------------------

FIX_SHIFT = 32     # u = rint(x * 2^32)
GAMMA_SHIFT = 24   # G = rint(gamma * 2^24)


def gamma_fixed(gamma: float) -> int:
    g32 = float(np.float32(gamma))
    return int(round(g32 * 2 ** GAMMA_SHIFT))


def select_cumulative(values: np.ndarray, gamma: float) -> np.ndarray:
    """Smallest set of entries whose summed value reaches gamma of the total.

    Values are float32 >= 0.  Each becomes u = rint(x * 2^32) as an integer;
    U = sum(u); T = ceil(G * U / 2^24) with G = rint(gamma * 2^24).  Entries
    are ordered by value descending, then index ascending; the selection is
    the shortest prefix of that order whose u-sum is >= T.  Returns a boolean
    mask over the entries."""
    x = np.asarray(values, dtype=F32)
    u = np.rint(x * F32(2.0 ** FIX_SHIFT)).astype(np.uint64)
    U = int(u.sum(dtype=np.uint64))
    G = gamma_fixed(gamma)
    T = (G * U + (1 << GAMMA_SHIFT) - 1) >> GAMMA_SHIFT
    sel = np.zeros(x.shape, dtype=bool)
    if T == 0:
        return sel
    order = np.argsort(-x, kind="stable")
    cs = np.cumsum(u[order], dtype=np.uint64)
    kk = int(np.searchsorted(cs, np.uint64(T), side="left"))
    sel[order[: kk + 1]] = True
    return sel


def vs_block_mask(sel_cols: np.ndarray, sel_diags: np.ndarray, bs: int) -> np.ndarray:
    """Selected vertical columns and slash offsets -> causal block mask.

    Any-touch rule (the block kernel computes whole blocks): block (qb, kb) is
    computed iff it contains at least one query/key pair (i, j), j <= i < N,
    with j selected or i - j selected.  Closed form: column j touches
    kb = j // bs in every row qb >= kb; offset o = a*bs + r touches the block
    diagonals qb - kb = a + 1 when r > 0 and qb - kb = a when r < tail(qb),
    where tail(qb) is the number of query rows of block row qb (bs except
    for a partial last block, N - (nb-1) bs)."""
    N = sel_cols.shape[0]
    nb = -(-N // bs)
    tail = N - (nb - 1) * bs
    col = np.zeros(nb, dtype=bool)
    col[np.nonzero(sel_cols)[0] // bs] = True
    o = np.nonzero(sel_diags)[0]
    dA = np.zeros(nb + 1, dtype=bool)          # some offset in diagonal a (any r)
    dA[o // bs] = True
    dT = np.zeros(nb + 1, dtype=bool)          # some offset in diagonal a with r < tail
    dT[o[o % bs < tail] // bs] = True
    dB = np.zeros(nb + 1, dtype=bool)          # some offset in diagonal a - 1 with r > 0
    dB[(o[o % bs > 0] // bs) + 1] = True
    qb = np.arange(nb)[:, None]
    kb = np.arange(nb)[None, :]
    dist = np.clip(qb - kb, 0, nb)
    own = np.where(qb == nb - 1, dT[dist], dA[dist])
    return (kb <= qb) & (col[kb] | own | dB[dist])


def tri_values(A: np.ndarray) -> np.ndarray:
    """The causal entries of a block map flattened row-major: index
    qb (qb + 1) / 2 + kb for kb <= qb (the ablation table's default: the
    estimated map is flattened into one list)."""
    r, c = np.tril_indices(A.shape[0])
    return A[r, c]


def qa_block_mask(sel_tri: np.ndarray, nb: int) -> np.ndarray:
    mask = np.zeros((nb, nb), dtype=bool)
    r, c = np.tril_indices(nb)
    mask[r[sel_tri], c[sel_tri]] = True
    return mask


def qa_querywise_mask(A: np.ndarray, gamma: float) -> np.ndarray:
    """Query-wise variant of the query-aware selection (an ablation-table
    alternative to selecting over the flattened map): every query-block row
    qb selects on its own, from its estimated row A[qb, 0..qb], the minimal
    set of key blocks whose mass reaches gamma of that row's total, with the
    same fixed-point test and tie order (value descending, key block
    ascending)."""
    nb = A.shape[0]
    mask = np.zeros((nb, nb), dtype=bool)
    for qb in range(nb):
        mask[qb, : qb + 1] = select_cumulative(A[qb, : qb + 1], gamma)
    return mask


def floor_blocks(min_budget: int, bs: int) -> int:
    """Blocks per query-block row that the minimum budget (in tokens, ablation
    table) asks for; every row keeps at least its diagonal block."""
    return max(1, -(-int(min_budget) // bs))


def apply_floor(mask: np.ndarray, min_budget: int, bs: int) -> np.ndarray:
    """Top each row qb up to min(qb + 1, floor) blocks, adding unselected
    blocks nearest-first (kb = qb, qb - 1, ...)."""
    mask = mask.copy()
    nb = mask.shape[0]
    f = floor_blocks(min_budget, bs)
    for qb in range(nb):
        want = min(qb + 1, f)
        have = int(mask[qb, : qb + 1].sum())
        kb = qb
        while have < want:
            if not mask[qb, kb]:
                mask[qb, kb] = True
                have += 1
            kb -= 1
    return mask


def cap_blocks(max_budget: int, bs: int) -> int:
    """Blocks per query-block row the maximum budget (tokens) allows; 0 means
    uncapped (the pages' default, ablation table)."""
    return 0 if max_budget <= 0 else -(-int(max_budget) // bs)


def vs_block_scores(c: np.ndarray, g: np.ndarray, sel_cols: np.ndarray, sel_diags: np.ndarray,
                    bs: int) -> np.ndarray:
    """Line mass a vertical-slash selection carries through each block:
    score(qb, kb) = colmass[kb] + diagmass[qb - kb], where colmass[kb] is the
    sum of the selected column scores c[j] in key block kb and diagmass[a] the
    sum of the selected diagonal scores g[o] whose offset touches block
    diagonal a (o // bs == a, or o // bs == a - 1 with o % bs > 0).  Sums in
    float32, ascending index.  The partial last row of a ragged sequence uses
    the same per-diagonal masses (a score, not an exact touch count)."""
    N = c.shape[0]
    nb = -(-N // bs)
    colmass = np.zeros(nb, dtype=F32)
    diagmass = np.zeros(nb + 1, dtype=F32)
    for j in np.nonzero(sel_cols)[0]:
        colmass[j // bs] = colmass[j // bs] + c[j]
    for o in np.nonzero(sel_diags)[0]:
        a = o // bs
        diagmass[a] = diagmass[a] + g[o]
    for o in np.nonzero(sel_diags)[0]:
        if o % bs > 0:
            diagmass[o // bs + 1] = diagmass[o // bs + 1] + g[o]
    qb = np.arange(nb)[:, None]
    kb = np.arange(nb)[None, :]
    return (colmass[kb] + diagmass[np.clip(qb - kb, 0, nb)]).astype(F32)


def apply_cap(mask: np.ndarray, scores: np.ndarray, max_budget: int, bs: int) -> np.ndarray:
    """Keep at most cap_blocks(max_budget) blocks per query-block row: the
    row's blocks ordered by score descending, then key block descending
    (nearest the diagonal first); the first `cap` of them stay."""
    cap = cap_blocks(max_budget, bs)
    if cap == 0:
        return mask
    mask = mask.copy()
    for qb in range(mask.shape[0]):
        kbs = np.nonzero(mask[qb, : qb + 1])[0]
        if len(kbs) <= cap:
            continue
        order = sorted(kbs.tolist(), key=lambda kb: (-float(scores[qb, kb]), -kb))
        mask[qb, :] = False
        mask[qb, order[:cap]] = True
    return mask


# --------------------------------------------------------------------------
# A whole head's plan.
# --------------------------------------------------------------------------

QUERY_AWARE = 1
VERTICAL_SLASH = 0


@dataclass
class HeadPlan:
    qbar: np.ndarray
    kbar: np.ndarray
    stats: LastBlockStats
    A: np.ndarray                # [nb, nb] estimated map (0 above the diagonal)
    jsd: float
    D: float
    pattern: int                 # QUERY_AWARE or VERTICAL_SLASH
    sel_qa: Optional[np.ndarray]
    sel_v: Optional[np.ndarray]
    sel_s: Optional[np.ndarray]
    mask: np.ndarray             # [nb, nb] final block mask incl. the floor
    lists: List[np.ndarray] = field(default_factory=list)
    cols: Optional[np.ndarray] = None   # [N] token-granular columns (vertical-slash, token mode)

    @property
    def counts(self) -> np.ndarray:
        return np.array([len(x) for x in self.lists], dtype=np.int64)


QA_FLATTENED = "flattened"
QA_QUERYWISE = "querywise"
VS_BLOCK = "block"
VS_TOKEN = "token"


def plan_head(q: np.ndarray, k: np.ndarray, bs: int, gamma: float, tau: float,
              min_budget: int, max_budget: int = 0, qa_selection: str = QA_FLATTENED,
              vs_granularity: str = VS_BLOCK) -> HeadPlan:
    """Pattern determination and index selection for one query head q [N, d]
    against its key/value head's keys k [N, d]; max_budget > 0 caps every
    query-block row (applied after the minimum-budget fill); qa_selection
    picks the flattened (default) or the query-wise selection for a
    query-aware head.

    vs_granularity = "token" keeps a vertical-slash head's selected key
    columns as single tokens instead of whole blocks: the block mask then
    holds the blocks its slash lines touch plus the minimum-budget fill (and
    the cap), and ``cols`` marks the columns every later query attends to
    individually (the pages call the selections lines; the blocked kernel is
    the default)."""
    if qa_selection not in (QA_FLATTENED, QA_QUERYWISE):
        raise ValueError(f"unknown qa_selection {qa_selection!r}")
    if vs_granularity not in (VS_BLOCK, VS_TOKEN):
        raise ValueError(f"unknown vs_granularity {vs_granularity!r}")
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    N, d = q.shape
    if N < 1:
        raise ValueError("a head needs at least one token")
    nb = -(-N // bs)
    qbar = pool_mean(q, bs)
    kbar = pool_mean(k, bs)
    st = last_block_stats(q, k, bs)
    A = estimate_map(qbar, kbar)
    jsd, D = jsd_canonical(A[nb - 1], st.a_true)
    pattern = QUERY_AWARE if D < float(np.float32(tau)) else VERTICAL_SLASH
    sel_qa = sel_v = sel_s = None
    if gamma_fixed(gamma) >= (1 << GAMMA_SHIFT):
        mask = np.tril(np.ones((nb, nb), dtype=bool))
    elif pattern == QUERY_AWARE and qa_selection == QA_QUERYWISE:
        mask = qa_querywise_mask(A, gamma)
        sel_qa = tri_values(mask)
    elif pattern == QUERY_AWARE:
        sel_qa = select_cumulative(tri_values(A), gamma)
        mask = qa_block_mask(sel_qa, nb)
    else:
        sel_v = select_cumulative(st.c, gamma)
        sel_s = select_cumulative(st.g, gamma)
        if vs_granularity == VS_TOKEN:
            mask = vs_block_mask(np.zeros_like(sel_v), sel_s, bs)
        else:
            mask = vs_block_mask(sel_v, sel_s, bs)
    mask = apply_floor(mask, min_budget, bs)
    if cap_blocks(max_budget, bs):
        if pattern == QUERY_AWARE or sel_v is None:
            scores = A
        else:
            scores = vs_block_scores(st.c, st.g, sel_v, sel_s, bs)
        mask = apply_cap(mask, scores, max_budget, bs)
    lists = [np.nonzero(mask[qb, : qb + 1])[0].astype(np.int32) for qb in range(nb)]
    cols = sel_v.copy() if (vs_granularity == VS_TOKEN and sel_v is not None) else None
    return HeadPlan(qbar, kbar, st, A, jsd, D, pattern, sel_qa, sel_v, sel_s, mask, lists, cols)


# --------------------------------------------------------------------------
# Step 3: attention restricted to the selected blocks (plain definition).
# --------------------------------------------------------------------------


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                bs: int, qbs: Iterable[int], cols: Optional[np.ndarray] = None) -> Dict[int, np.ndarray]:
    """float64 attention outputs of the query blocks ``qbs``: for query i the
    keys j <= i whose block (i // bs, j // bs) is in ``mask`` or, when given,
    whose column is marked in ``cols``; scores q_i . k_j / sqrt(d); softmax;
    weighted sum of v_j.  A partial last block (N not a multiple of bs) has
    N - qb bs rows."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    N, d = q.shape
    out = {}
    for qb in qbs:
        end = min(N, (qb + 1) * bs)
        i = np.arange(qb * bs, end)
        s = (q[i] @ k[:end].T) / math.sqrt(d)
        j = np.arange(end)
        sel = mask[qb, j // bs]
        if cols is not None:
            sel = sel | cols[:end]
        keep = (j[None, :] <= i[:, None]) & sel[None, :]
        s = np.where(keep, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        w = np.where(keep, np.exp(s - mx), 0.0)
        w /= w.sum(axis=1, keepdims=True)
        out[qb] = w @ v[:end]
    return out


def attend_head(q, k, v, mask, bs, cols=None) -> np.ndarray:
    nb = -(-q.shape[0] // bs)
    rows = attend_rows(q, k, v, mask, bs, range(nb), cols)
    return np.concatenate([rows[qb] for qb in range(nb)], axis=0)


def dense_mask(nb: int) -> np.ndarray:
    return np.tril(np.ones((nb, nb), dtype=bool))
