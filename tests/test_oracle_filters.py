"""Pins for the oracle's filter chain (top-k, top-p, min-p) and its use in the verify rule.

mlxcel PR #992, section What changed, names the chain: temperature scale,
top-k, top-p, min-p, then the softmax of what is left. What fixes the answers
here lies outside ``oracle.filters``:

* Hand-worked examples on p = (1/2, 1/4, 1/8, 1/16, 1/16). Their kept sets
  follow from the definitions by mental arithmetic. One of them tells "top-p on
  top-k's renormalised set" apart from "top-p on the full distribution".
* Brute force on tiny rows: an exhaustive search over every subset of tokens
  that the readings allow as a kept set. It shares no step with the oracle's
  sort-and-cumulate.
* Invariants of the definitions on random rows: settings that turn a filter off
  change nothing, and the kept sets are monotone in each parameter. The kept
  top-p mass reaches top_p, and it falls below top_p without the smallest
  kept value. Ties at a threshold are kept.
* The page's zero-tolerance property (section Where chi-square is blind): a
  top_k = 2 target against an unfiltered drafter never emits a token outside
  the target's two-token support, over at least 1500 emitted tokens. The same
  inputs without the target filter do emit such tokens, so the check has
  power.
* Losslessness with filtered p and q: the first emitted token follows the
  filtered target law (chi-square at alpha 1e-4). scipy's softmax of the
  kept logits supplies the law.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import filters as of
from oracle import verify as ov
from tests.helpers import batch_from_rows, chi2_threshold, chi_square

P5 = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
X5 = np.log(P5)


def kept(x, T, f):
    theta, _ = of.threshold(x, T, f)
    return {i for i in range(x.size) if x[i] >= theta}


# ---------------------------------------------------------------- hand-worked examples

@pytest.mark.parametrize("k, want", [(1, {0}), (2, {0, 1}), (3, {0, 1, 2}),
                                     (4, {0, 1, 2, 3, 4}),   # the 4th and 5th tie: both kept
                                     (5, {0, 1, 2, 3, 4}), (0, {0, 1, 2, 3, 4})])
def test_top_k_by_hand(k, want):
    assert kept(X5, 1.0, of.Filter(top_k=k)) == want


@pytest.mark.parametrize("tp, want", [(0.4, {0}), (0.7, {0, 1}), (0.8, {0, 1, 2}),
                                      (0.9, {0, 1, 2, 3, 4}),  # crosses inside the tied pair
                                      (1.0, {0, 1, 2, 3, 4})])
def test_top_p_by_hand(tp, want):
    assert kept(X5, 1.0, of.Filter(top_p=tp)) == want


def test_top_p_works_on_top_k_renormalised_set():
    # top-3 leaves (4/7, 2/7, 1/7): top_p 0.8 is reached by 6/7 with two tokens. On the full
    # distribution the two-token prefix holds only 3/4 and a third token would be needed.
    assert kept(X5, 1.0, of.Filter(top_k=3, top_p=0.8)) == {0, 1}
    assert kept(X5, 1.0, of.Filter(top_p=0.8)) == {0, 1, 2}


@pytest.mark.parametrize("T, mp, want", [(1.0, 0.3, {0, 1}), (1.0, 0.2, {0, 1, 2}), (1.0, 1.0, {0}),
                                         # at T = 2 the ratios to the max are sqrt(p / 0.5)
                                         (2.0, 0.45, {0, 1, 2}), (2.0, 0.55, {0, 1}),
                                         (2.0, 0.35, {0, 1, 2, 3, 4})])  # sqrt(1/8) = 0.354
def test_min_p_by_hand(T, mp, want):
    assert kept(X5, T, of.Filter(min_p=mp)) == want


def test_filtered_probabilities_by_hand():
    p, near = of.filtered_distribution(X5, 1.0, of.Filter(top_k=2))
    assert not near
    assert np.allclose(p, [2 / 3, 1 / 3, 0, 0, 0], rtol=1e-15, atol=0)
    p, _ = of.filtered_distribution(X5, 1.0, of.Filter(top_p=0.8, min_p=0.3))  # min-p binds
    assert np.allclose(p, [2 / 3, 1 / 3, 0, 0, 0], rtol=1e-15, atol=0)


def test_chain_with_all_three_takes_the_tightest():
    assert kept(X5, 1.0, of.Filter(top_k=4, top_p=0.9, min_p=0.2)) == {0, 1, 2}


# ---------------------------------------------------------------- brute force on tiny rows

def _brute_kept(x, T, f):
    """Kept set by exhaustive search, from the readings, with no sorting or prefix sums."""
    V = x.size
    idx = range(V)
    m = max(x)
    e = [math.exp((x[i] - m) / T) for i in idx]

    def upward_closed(S):
        # with every token of S, every token with an equal or larger logit is in S
        return all(x[j] < x[i] for i in S for j in idx if j not in S)

    subsets = [frozenset(c) for n in range(1, V + 1) for c in itertools.combinations(idx, n)]
    closed = [S for S in subsets if upward_closed(S)]
    # top-k: the smallest closed set holding at least k tokens
    if 0 < f.top_k < V:
        Sk = min((S for S in closed if len(S) >= f.top_k), key=len)
    else:
        Sk = frozenset(idx)
    Sp = Sk
    if f.top_p < 1.0:
        S1 = sum(e[i] for i in Sk)
        Sp = min((S for S in closed if S <= Sk and sum(e[i] for i in S) >= f.top_p * S1), key=len)
    Sm = frozenset(idx)
    if f.min_p > 0.0:
        Sm = frozenset(i for i in idx if (x[i] - m) / T >= math.log(f.min_p))
    return set(Sp & Sm)


def test_matches_brute_force_on_tiny_rows():
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(600):
        V = int(rng.integers(2, 8))
        x = rng.integers(-6, 7, size=V) / 2.0   # a coarse lattice makes ties common
        T = float(rng.choice([0.5, 1.0, 1.7]))
        f = of.Filter(top_k=int(rng.integers(0, V + 1)),
                      top_p=float(rng.choice([1.0, 0.3, 0.55, 0.77, 0.93])),
                      min_p=float(rng.choice([0.0, 0.05, 0.21, 0.6])))
        theta, near = of.threshold(x, T, f)
        if near:
            continue
        assert kept(x, T, f) == _brute_kept(x, T, f), (x, T, f)
        checked += 1
    assert checked > 500


# ---------------------------------------------------------------- invariants on random rows

def _row(rng, V=4000, sigma=3.0):
    return rng.normal(0, sigma, size=V).astype(np.float32).astype(np.float64)


def test_settings_that_turn_filters_off_change_nothing():
    rng = np.random.default_rng(1)
    x = _row(rng)
    want = sp_softmax(x / 0.8)
    for f in (of.Filter(), of.Filter(top_k=x.size), of.Filter(top_k=x.size + 7), of.Filter(top_p=1.0),
              of.Filter(top_p=1.5), of.Filter(min_p=0.0)):
        p, near = ov.row_distribution(x, 0.8, f)
        assert not near
        assert np.allclose(p, want, rtol=1e-12, atol=0)


def test_kept_sets_are_monotone_and_top_p_is_minimal():
    rng = np.random.default_rng(2)
    for trial in range(6):
        x = _row(rng)
        T = [0.6, 1.0, 1.3][trial % 3]
        prev = None
        for k in (1, 5, 50, 400, 3999):
            s = kept(x, T, of.Filter(top_k=k))
            assert len(s) >= k
            assert prev is None or prev <= s
            prev = s
        prev = None
        e = np.exp((x - x.max()) / T)
        for tp in (0.1, 0.5, 0.9, 0.99):
            theta, near = of.threshold(x, T, of.Filter(top_p=tp))
            assert not near
            s = x >= theta
            assert e[s].sum() >= tp * e.sum()
            without = x > theta  # drop the smallest kept value (and its ties)
            assert e[without].sum() < tp * e.sum()
            assert prev is None or (prev & ~s).sum() == 0
            prev = s
        prev = None
        for mp in (0.001, 0.05, 0.5, 1.0):
            s = kept(x, T, of.Filter(min_p=mp))
            assert int(np.argmax(x)) in s
            assert prev is None or s <= prev
            prev = s


def test_ties_at_the_threshold_are_kept():
    x = np.array([3.0, 1.0, 1.0, 1.0, 0.0, -2.0])
    assert kept(x, 1.0, of.Filter(top_k=2)) == {0, 1, 2, 3}
    assert kept(x, 1.0, of.Filter(top_k=1)) == {0}
    x = np.array([2.0, 2.0, 0.0])
    assert kept(x, 1.0, of.Filter(top_k=1)) == {0, 1}   # a tied maximum: both kept


def test_near_band_flags_top_p_and_min_p():
    # mass 1/2 on token 0: top_p = 0.5 sits exactly on the boundary
    _, near = of.threshold(X5, 1.0, of.Filter(top_p=0.5))
    assert near
    _, near = of.threshold(X5, 1.0, of.Filter(top_p=0.5 + 1e-3))
    assert not near
    _, near = of.threshold(X5, 1.0, of.Filter(min_p=0.25))  # token 2 has ratio exactly 1/4
    assert near


def test_invalid_filter_fails_the_request_and_greedy_ignores_it():
    x = np.log(np.array([[0.6, 0.3, 0.1], [0.6, 0.3, 0.1]]))
    dt = np.array([0, -1])
    for bad in (of.Filter(top_k=-1), of.Filter(top_p=0.0), of.Filter(top_p=float("nan")),
                of.Filter(min_p=1.5), of.Filter(min_p=-0.1)):
        assert ov.verify_request(x, x, dt, 1.0, 0.0, 1, 0, tfilt=bad).accept_len == -1
        assert ov.verify_request(x, x, dt, 1.0, 0.0, 1, 0, dfilt=bad).accept_len == -1
        assert ov.verify_request(x, x, dt, 0.0, 0.0, 1, 0, tfilt=bad).accept_len == 1


# ---------------------------------------------------------------- the verify rule with filters

def _support_batch(rng, n_req, V=8, n_draft=3, T=1.0):
    rows = n_draft + 1
    R = n_req * rows
    tl = rng.normal(0, 1.5, size=(R, V)).astype(np.float32)
    dl = rng.normal(0, 1.5, size=(R, V)).astype(np.float32)
    toks = np.empty(R, dtype=np.int64)
    for r in range(R):   # the drafter samples its own unfiltered q
        toks[r] = rng.choice(V, p=sp_softmax(dl[r].astype(np.float64) / T))
    toks[rows - 1::rows] = -1
    ro = np.arange(0, R + 1, rows)
    return batch_from_rows(tl, dl, toks, ro, np.full(n_req, T), np.zeros(n_req)), rows


def test_filtered_target_support_is_never_violated():
    rng = np.random.default_rng(7)
    batch, rows = _support_batch(rng, 1200)
    B = len(batch["row_offsets"]) - 1
    tf = (np.full(B, 2, dtype=np.int32), None, None)
    res = ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                          batch["temperature"], batch["tau"], 11, "f32", target_filter=tf)
    n = 0
    unfiltered_outside = 0
    res0 = ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                           batch["temperature"], batch["tau"], 11, "f32")
    for b in range(B):
        lo = b * rows
        k = int(res.out_accept_len[b])
        assert k >= 0
        for j in range(k + 1):
            top2 = set(np.argsort(-batch["target"][lo + j].astype(np.float64))[:2].tolist())
            assert int(res.out_tokens[lo + j]) in top2
            n += 1
        k0 = int(res0.out_accept_len[b])
        for j in range(k0 + 1):
            top2 = set(np.argsort(-batch["target"][lo + j].astype(np.float64))[:2].tolist())
            unfiltered_outside += int(res0.out_tokens[lo + j]) not in top2
    assert n >= 1500
    assert unfiltered_outside > 100   # without the filter such tokens are common


def test_first_token_follows_the_filtered_target_law():
    V, T, n_req, n_draft = 6, 0.9, 12000, 1
    t_log = np.array([2.0, 1.5, 1.2, 0.3, -0.4, -1.0], dtype=np.float32)
    d_log = np.array([0.5, 1.9, 1.0, 1.1, 0.2, -0.3], dtype=np.float32)
    tf_ = of.Filter(top_k=4, top_p=0.95)
    df_ = of.Filter(top_p=0.9, min_p=0.1)
    # The target law from scipy's softmax: top-4 keeps tokens 0..3; top-p then keeps the
    # fewest of them, by decreasing logit, whose renormalised mass reaches 0.95.
    t64 = t_log.astype(np.float64)
    d64 = d_log.astype(np.float64)
    keep_t = np.array([1, 1, 1, 1, 0, 0], dtype=bool)
    pt = np.zeros(V)
    pt[keep_t] = sp_softmax(t64[keep_t] / T)
    c = np.cumsum(np.sort(pt)[::-1])
    n_keep = int(np.argmax(c >= 0.95)) + 1
    order = np.argsort(-t64)
    keep_t = np.zeros(V, dtype=bool)
    keep_t[order[:n_keep]] = True
    p_law = np.zeros(V)
    p_law[keep_t] = sp_softmax(t64[keep_t] / T)
    q_full = sp_softmax(d64 / T)
    assert set(np.flatnonzero(keep_t)) == set(np.flatnonzero(ov.row_distribution(t64, T, tf_)[0]))

    rng = np.random.default_rng(3)
    q_draw, _ = ov.row_distribution(d64, T, df_)   # the drafter draws from its filtered q
    assert np.count_nonzero(q_draw) < V and np.isclose(q_draw[q_draw > 0].sum(), 1.0)
    rows = n_draft + 1
    R = n_req * rows
    toks = rng.choice(V, size=R, p=q_draw)
    toks[rows - 1::rows] = -1
    batch = batch_from_rows(np.tile(t_log, (R, 1)), np.tile(d_log, (R, 1)), toks, np.arange(0, R + 1, rows),
                            np.full(n_req, T), np.zeros(n_req))
    tf = (np.full(n_req, tf_.top_k, np.int32), np.full(n_req, tf_.top_p, np.float32), None)
    df = (None, np.full(n_req, df_.top_p, np.float32), np.full(n_req, df_.min_p, np.float32))
    res = ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                          batch["temperature"], batch["tau"], 5, "f32", target_filter=tf, draft_filter=df)
    first = res.out_tokens[0::rows]
    assert (res.out_accept_len >= 0).all()
    stat = chi_square(first.astype(np.int64), p_law)
    dof = int(np.count_nonzero(p_law)) - 1
    assert stat < chi2_threshold(dof, 1e-4), stat
    assert q_full.min() > 0  # the drafter's unfiltered law has full support; the filter removed some


def test_flag_band_ignores_decisions_that_are_exact():
    # min_p = 1 keeps exactly the maximum's ties; a crossing at the largest value has no
    # larger value to compare with.
    _, near = of.threshold(X5, 1.0, of.Filter(min_p=1.0))
    assert not near
    _, near = of.threshold(X5, 1.0, of.Filter(top_p=1e-6))
    assert not near
    assert kept(X5, 1.0, of.Filter(top_p=1e-6)) == {0}
    _, near = of.threshold(X5, 1.0, of.Filter(top_p=0.5))   # the largest value's mass is top_p
    assert near


# ---------------------------------------------------------------- bounds the GPU kernel relies on

def test_top_p_crossing_lies_inside_the_mass_window():
    # A logit more than W = log2(V / (1 - top_p)) + 1 log2 units of mass below the maximum
    # cannot be top-p's crossing: all such logits together hold under (1 - top_p) / 2 of the
    # row's mass. Checked against the oracle's threshold on peaked and flat rows.
    rng = np.random.default_rng(41)
    for trial in range(60):
        V = int(rng.choice([50, 1000, 20000]))
        sigma = float(rng.choice([0.3, 1.0, 3.0, 6.0]))
        x = rng.normal(0, sigma, size=V).astype(np.float32).astype(np.float64)
        if trial % 3 == 0:
            x[rng.integers(0, V, size=4)] += 8 * sigma
        T = float(rng.choice([0.5, 1.0, 1.3]))
        tp = float(np.float32(rng.choice([0.3, 0.9, 0.99, 0.9999])))
        theta, _ = of.threshold(x, T, of.Filter(top_p=tp))
        W = np.log2(V / (1.0 - tp)) + 1.0
        depth = (x.max() - theta) / T * np.log2(np.e)   # log2 units of mass below the maximum
        assert depth < W, (V, sigma, T, tp, depth, W)


def test_kth_largest_block_maximum_bounds_the_kth_largest_logit():
    # Split a row into blocks (the kernel's threads read strided blocks): at least k logits reach
    # the k-th largest block maximum, so it is at most the row's k-th largest logit.
    rng = np.random.default_rng(43)
    for _ in range(200):
        V = int(rng.integers(1, 5000))
        nb = int(rng.choice([7, 64, 512]))
        x = np.round(rng.normal(0, 2, size=V), 1)        # ties are common
        k = int(rng.integers(1, min(V, nb) + 1))
        owner = np.arange(V) % nb
        maxima = np.full(nb, -np.inf)
        np.maximum.at(maxima, owner, x)
        edge = np.sort(maxima)[::-1][k - 1]
        kth = np.sort(x)[::-1][k - 1]
        assert edge <= kth
        assert np.count_nonzero(x >= edge) >= k
