"""Pins for the oracle's per-row acceptance sums (oracle.verify.row_sums).

sum_x min(p, mu) is the probability that a row accepts its draft, given its
prefix (Strata PR #3416, section Approach; mlxcel PR #992, section The
acceptance ceiling); sum_x p q is the sampler-match rule's. Pins:
* the exact rational closed form of oracle.exact (itself pinned by exhaustive
  enumeration) on rational p, q given as logits;
* greedy rows: one-hot p and q give [argmax p = argmax q] for both sums, the
  first one also needing tau <= 1;
* which rows carry values: proposal rows only;
* the cumulative floor raises a later row's threshold from the drafted
  tokens' probabilities (regolith audit, section schedule behavior).
"""
from fractions import Fraction as F

import numpy as np

from oracle import exact
from oracle import verify as ov
from tests.helpers import batch_from_rows


def _logits(law):
    return np.log(np.array([float(x) for x in law], dtype=np.float64))


def _sums(rows_t, rows_d, dt, T, tau, **kw):
    b = batch_from_rows(rows_t, rows_d, dt, [0, len(dt)], [T], [tau])
    smin, spq, _ = ov.row_sums(b["target"], b["draft"], b["draft_tokens"], b["row_offsets"], b["temperature"],
                               b["tau"], "f32", **kw)
    return smin, spq


def test_matches_exact_closed_form():
    laws = [lw for lw in exact.all_rational_laws(3, 6) if all(x > 0 for x in lw)]
    rng = np.random.default_rng(5)
    for _ in range(40):
        p = laws[rng.integers(len(laws))]
        q = laws[rng.integers(len(laws))]
        tau = [F(0), F(1, 6), F(1, 3), F(1, 2)][rng.integers(4)]
        # q's entries are multiples of 1/6 and tau sits exactly on the grid: nudge tau below a grid
        # point by far more than fp32 rounding so that the gate decision is the exact one
        tau_f = float(tau) - 1e-4 if tau > 0 else 0.0
        t = np.stack([_logits(p), _logits(p)])
        d = np.stack([_logits(q), _logits(q)])
        smin, spq = _sums(t, d, [0, -1], 1.0, tau_f)
        want_min = exact.acceptance_probability(p, q, tau - F(1, 10000) if tau > 0 else F(0))
        want_pq = sum(a * b for a, b in zip(p, q))
        assert abs(smin[0] - float(want_min)) < 1e-6
        assert abs(spq[0] - float(want_pq)) < 1e-6
        assert np.isnan(smin[1]) and np.isnan(spq[1])


def test_greedy_rows():
    t = np.array([[0.0, 3.0, 1.0], [0.0, 3.0, 1.0], [1.0, 0.0, 0.0]])
    d = np.array([[0.0, 2.0, 1.0], [5.0, 2.0, 1.0], [0.0, 0.0, 0.0]])
    smin, spq = _sums(t, d, [1, 0, -1], 0.0, 0.5)
    assert smin[0] == 1.0 and spq[0] == 1.0      # same argmax
    assert smin[1] == 0.0 and spq[1] == 0.0      # different argmax
    smin, _ = _sums(t, d, [1, 0, -1], 0.0, 1.5)
    assert smin[0] == 0.0                        # tau > 1 gates the one-hot q away


def test_only_proposal_rows_carry_values():
    t = np.zeros((5, 4))
    smin, spq = _sums(t, t, [1, 2, -1, 3, 0], 1.0, 0.0)
    assert np.all(np.isfinite(smin[:2])) and np.all(np.isnan(smin[2:]))
    assert np.allclose(smin[:2], 1.0) and np.allclose(spq[:2], 0.25)


def test_cumulative_floor_raises_later_thresholds():
    # row 0: q(D=0) = 1/2; a floor of 0.4 gates row 1 at 0.8
    q0 = [F(1, 2), F(1, 4), F(1, 4)]
    q1 = [F(5, 6), F(1, 12), F(1, 12)]
    p1 = [F(1, 3), F(1, 3), F(1, 3)]
    t = np.stack([_logits(q0), _logits(p1), _logits(p1)])
    d = np.stack([_logits(q0), _logits(q1), _logits(q1)])
    smin, _ = _sums(t, d, [0, 0, -1], 1.0, 0.0, min_cum=np.array([0.4], dtype=np.float32))
    assert abs(smin[1] - float(exact.acceptance_probability(p1, q1, F(4, 5)))) < 1e-6
    smin0, _ = _sums(t, d, [0, 0, -1], 1.0, 0.0)
    assert abs(smin0[1] - float(exact.acceptance_probability(p1, q1, F(0)))) < 1e-6
    assert smin[1] < smin0[1]


def test_filtered_sums_match_the_exact_closed_form_on_filtered_laws():
    # p = (1/2, 1/4, 1/8, 1/16, 1/16) under top-k 2 is (2/3, 1/3, 0, 0, 0) exactly; q under
    # min-p 0.3 keeps the tokens with ratio >= 0.3 to its maximum. The exact closed form on
    # those filtered laws (oracle.exact) pins the filtered sums.
    p_law = [F(1, 2), F(1, 4), F(1, 8), F(1, 16), F(1, 16)]
    q_law = [F(1, 10), F(4, 10), F(3, 10), F(1, 10), F(1, 10)]
    p_f = [F(2, 3), F(1, 3), F(0), F(0), F(0)]
    q_f = [F(0), F(4, 7), F(3, 7), F(0), F(0)]    # ratios 1/4, 1, 3/4, 1/4, 1/4: keeps 1 and 2
    rows_t = np.stack([_logits(p_law), _logits(p_law)])
    rows_d = np.stack([_logits(q_law), _logits(q_law)])
    for tau in (0.0, 0.5):
        smin, spq = _sums(rows_t, rows_d, [1, -1], 1.0, tau,
                          target_filter=(np.array([2], np.int32), None, None),
                          draft_filter=(None, None, np.array([0.3], np.float32)))
        want = exact.acceptance_probability(p_f, q_f, F(tau).limit_denominator(10))
        assert abs(smin[0] - float(want)) < 1e-6    # the logits are stored in fp32
        assert abs(spq[0] - float(sum(a * b for a, b in zip(p_f, q_f)))) < 1e-6
        assert np.isnan(smin[1])
    # an invalid filter value fails the request: NaN
    smin, _ = _sums(rows_t, rows_d, [1, -1], 1.0, 0.0, target_filter=(np.array([-1], np.int32), None, None))
    assert np.isnan(smin[0])
