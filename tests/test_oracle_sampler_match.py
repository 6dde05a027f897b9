"""Pins for the oracle's sampler-match rule (mlxcel PR #992, sections The premise
correction and The acceptance ceiling).

The rule accepts a drafted token iff it equals a fresh draw from the target
and emits that draw on both branches. What fixes the answer:

* Exact enumeration (rationals, V <= 4): the emitted token's law is p for
  every p and q, the acceptance is sum_x p(x) q(x), and it never exceeds the
  method's sum_x min(p, q) (the acceptance ceiling's table and its min >= product
  argument). Whole windows: every position's token is p-distributed and the
  window's law factors row by row.
* The page's chi-square recipe (6 tokens, T = 0.7, 12000 tokens, threshold
  25.7448): sampler-match passes it, as the page reports.
* The sampled acceptance frequency sits on sum_x p(x) q(x), measurably below
  the method's sum_x min(p, q) on the same rows.
* At T = 0 the rule is argmax-against-argmax, bit for bit.
* The draws do not depend on the drafted tokens: feeding a run's own emitted
  tokens back as the drafts accepts every row and emits the same tokens.
"""
import json
import os
from fractions import Fraction as F
from itertools import product

import numpy as np
import pytest

from oracle import exact
from oracle import verify as ov
from tests.helpers import chi_square, emitted_tokens, repeated_window, target_law

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CHI_T = [1.2, 0.4, -0.3, 0.9, -1.1, 0.0]
CHI_D = [0.2, 1.1, -0.5, 0.3, 0.6, -0.9]


def _run(batch, rule, requests=None):
    return ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                           batch["temperature"], batch["tau"], batch["seed"], batch["dtype"],
                           requests=requests, rule=rule)


@pytest.mark.parametrize("V,denom", [(2, 8), (3, 5), (4, 3)])
def test_exact_marginal_and_acceptance(V, denom):
    laws = list(exact.all_rational_laws(V, denom))
    for p, q in product(laws, laws):
        accepted, fallback = exact.row_law(p, q, F(0), "sampler_match")
        assert [a + f for a, f in zip(accepted, fallback)] == p
        acc = sum(accepted)
        assert acc == sum(a * b for a, b in zip(p, q))
        assert acc <= exact.acceptance_probability(p, q, F(0))
        # the gate plays no part in this rule
        assert exact.row_law(p, q, F(1, 2), "sampler_match") == (accepted, fallback)


def test_exact_window_positions_are_p_distributed():
    ps = [[F(1, 2), F(1, 3), F(1, 6)], [F(1, 5), F(3, 5), F(1, 5)], [F(1, 4), F(1, 4), F(1, 2)]]
    qs = [[F(2, 3), F(1, 6), F(1, 6)], [F(0), F(1, 2), F(1, 2)]]
    law = exact.window_law(ps, qs, F(0), "sampler_match")
    assert sum(law.values()) == 1
    for pos in range(3):
        marg = [F(0)] * 3
        reach = F(0)
        for (k, toks), pr in law.items():
            if len(toks) > pos:
                marg[toks[pos]] += pr
                reach += pr
        assert [m / reach for m in marg] == ps[pos]
    # P(accept_len >= 1) = sum p0 q0; P(accept_len = 2) = (sum p0 q0)(sum p1 q1)
    a0 = sum(a * b for a, b in zip(ps[0], qs[0]))
    a1 = sum(a * b for a, b in zip(ps[1], qs[1]))
    assert sum(pr for (k, _), pr in law.items() if k >= 1) == a0
    assert sum(pr for (k, _), pr in law.items() if k == 2) == a0 * a1


def test_chi_square_sampler_match_passes(stat_samples):
    g = json.load(open(os.path.join(GOLD, "chi_square.json")))
    T = g["temperature"]
    p = target_law(CHI_T, T)
    batch = repeated_window(CHI_T, CHI_D, stat_samples + 50, 4, T, 0.0, np.random.default_rng(5), seed=55)
    res = _run(batch, "sampler_match")
    toks = emitted_tokens(res.out_tokens, res.out_accept_len, batch["row_offsets"])[:stat_samples]
    assert toks.size == stat_samples
    chi = chi_square(toks, p)
    assert chi < g["threshold"], chi


def test_acceptance_frequency_is_sum_pq():
    T = 0.9
    p = target_law(CHI_T, T)
    q = target_law(CHI_D, T)
    spq = float((p * q).sum())
    smin = float(np.minimum(p, q).sum())
    n = 20000
    batch = repeated_window(CHI_T, CHI_D, n, 1, T, 0.0, np.random.default_rng(9), seed=91)
    acc = float((_run(batch, "sampler_match").out_accept_len == 1).mean())
    sd = np.sqrt(spq * (1 - spq) / n)
    assert abs(acc - spq) < 4.5 * sd, (acc, spq)
    assert smin - spq > 20 * sd  # the method's ceiling is well separated on these rows
    acc_mu = float((_run(batch, "mu").out_accept_len == 1).mean())
    assert acc_mu - acc > 10 * sd, (acc_mu, acc)


def test_greedy_is_argmax_against_argmax():
    rng = np.random.default_rng(3)
    batch = repeated_window(CHI_T, CHI_D, 200, 3, 0.0, 0.0, rng)
    # vary the rows so that some drafts match the target's argmax and some do not
    batch["target"] = rng.normal(0, 1, size=batch["target"].shape).astype(np.float32)
    batch["draft_tokens"] = np.where(batch["draft_tokens"] >= 0,
                                     rng.integers(0, 2, size=batch["draft_tokens"].shape) *
                                     np.argmax(batch["target"], axis=1), -1).astype(np.int32)
    a = _run(batch, "sampler_match")
    b = _run(batch, "argmax")
    assert np.array_equal(a.out_tokens, b.out_tokens)
    assert np.array_equal(a.out_accept_len, b.out_accept_len)
    assert (a.out_accept_len > 0).any() and (a.out_accept_len < 3).any()


def test_draws_do_not_depend_on_the_drafts():
    rng = np.random.default_rng(4)
    n_req, n_draft, V = 40, 5, 50
    batch = repeated_window(rng.normal(size=V), rng.normal(size=V), n_req, n_draft, 1.0, 0.0, rng, seed=21)
    batch["target"] = rng.normal(0, 0.5, size=batch["target"].shape).astype(np.float32)
    ro = batch["row_offsets"]
    # Feed back each request's emitted tokens as its drafts until every row is accepted.
    for _ in range(n_draft + 1):
        res = _run(batch, "sampler_match")
        for b in range(n_req):
            k = int(res.out_accept_len[b])
            lo = ro[b]
            if k < n_draft:
                batch["draft_tokens"][lo + k] = res.out_tokens[lo + k]
    final = _run(batch, "sampler_match")
    assert (final.out_accept_len == n_draft).all()
    for b in range(n_req):
        lo = ro[b]
        assert np.array_equal(final.out_tokens[lo:lo + n_draft], batch["draft_tokens"][lo:lo + n_draft])
