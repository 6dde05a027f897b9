"""Exact (rational) pins for the oracle's verify rule.

* The worked example printed in Strata PR #3416, section Problem and result:
  the original gate emits (0.5625, 0.4375) and the repaired rule emits
  exactly (0.5, 0.5).
* Losslessness, by exhaustive enumeration at V <= 4: the emitted token's law
  is exactly p. This holds for every rational p and q on a grid and every
  tau, including tau = 0 (ungated), tau = 1 and tau > 1.
* The accept probability equals sum_x min(p, mu). Ungated it equals
  1 - TV(p, q) (mlxcel PR #992, section The acceptance ceiling).
* sum min >= sum p*q (the same section), and the argmax example from that
  section.
* Prefix survival is a product of per-step acceptances (regolith audit,
  section economics and confidence), and each position's token is
  p-distributed.
"""
import json
import os
from fractions import Fraction as F
from itertools import product

import pytest

from oracle import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_example_both_rules():
    g = _gold("worked_example.json")
    p = [F(x) for x in g["p"]]
    q = [F(x) for x in g["q"]]
    tau = F(g["tau"])
    repaired = exact.first_token_distribution(p, q, tau, "mu")
    original = exact.first_token_distribution(p, q, tau, "original")
    assert [float(x) for x in repaired] == g["repaired_rule_emits"]
    assert [float(x) for x in original] == g["original_rule_emits"]
    assert repaired == [F(1, 2), F(1, 2)]
    assert original == [F(9, 16), F(7, 16)]


TAUS = [F(0), F(1, 10), F(1, 4), F(1, 3), F(1, 2), F(2, 3), F(1), F(3, 2)]


def _grid(V, denom):
    return list(exact.all_rational_laws(V, denom))


@pytest.mark.parametrize("V,denom", [(1, 1), (2, 8), (3, 5), (4, 3)])
def test_lossless_by_enumeration(V, denom):
    laws = _grid(V, denom)
    n = 0
    for p, q in product(laws, laws):
        for tau in TAUS:
            got = exact.first_token_distribution(p, q, tau, "mu")
            assert got == p, (p, q, tau, got)
            n += 1
    assert n > 0


def test_original_rule_is_biased_somewhere():
    laws = _grid(3, 4)
    biased = 0
    for p, q in product(laws, laws):
        for tau in TAUS[1:-1]:
            if exact.first_token_distribution(p, q, tau, "original") != p:
                biased += 1
    assert biased > 0
    # Ungated (tau = 0) the original rule is ordinary modified rejection sampling, hence lossless.
    for p, q in product(laws, laws):
        assert exact.first_token_distribution(p, q, F(0), "original") == p


def test_acceptance_probability_closed_form():
    laws = _grid(3, 6)
    for p, q in product(laws, laws):
        for tau in TAUS:
            accepted, _ = exact.row_law(p, q, tau, "mu")
            mu = exact.retained_measure(q, tau)
            assert sum(accepted) == sum(min(a, b) for a, b in zip(p, mu))
            # per token: P(accept and emit x) = min(p(x), mu(x))
            assert accepted == [min(a, b) for a, b in zip(p, mu)]
        # ungated: 1 - TV(p, q)
        tv = sum(abs(a - b) for a, b in zip(p, q)) / 2
        assert exact.acceptance_probability(p, q, F(0)) == 1 - tv


def test_sum_min_at_least_sum_prod_and_argmax_example():
    laws = _grid(4, 4)
    for p, q in product(laws, laws):
        assert sum(min(a, b) for a, b in zip(p, q)) >= sum(a * b for a, b in zip(p, q))
    g = _gold("acceptance_ceiling.json")
    # token a is the target's argmax with p(a) = 0.3; the draft puts q(a) = 0.95 on it.
    p = [F(3, 10), F(1, 4), F(1, 4), F(1, 5)]
    q = [F(95, 100), F(1, 60), F(1, 60), F(1, 60)]
    assert max(range(4), key=lambda x: p[x]) == 0 and max(range(4), key=lambda x: q[x]) == 0
    ceiling = sum(min(a, b) for a, b in zip(p, q))
    # argmax-against-argmax accepts whenever the draft draws a: probability q(a)
    assert float(q[0]) == g["argmax_rule_accepts"]
    # every lossless rule is capped by sum min(p, q), which lies in [p(a), p(a) + 1 - q(a)]
    assert F(3, 10) <= ceiling <= F(3, 10) + (1 - q[0])
    assert float(p[0]) == g["ceiling_about"]
    assert q[0] > ceiling


def test_prefix_survival_golden():
    g = _gold("prefix_survival.json")
    # rows with acceptance exactly 1/2 each: p = (1/2, 1/2), q = (1, 0) -> sum min = 1/2
    p = [F(1, 2), F(1, 2)]
    q = [F(1), F(0)]
    n = len(g["per_step_acceptance"]) + 1
    law = exact.window_law([p] * n, [q] * (n - 1), F(0))
    for i, want in enumerate(g["prefix_survival"], start=1):
        got = sum(pr for (k, _), pr in law.items() if k >= i)
        assert float(got) == want


def test_window_law_product_and_positionwise_marginals():
    laws3 = _grid(3, 4)
    import random
    rnd = random.Random(7)
    for _ in range(60):
        n = rnd.randint(2, 4)
        ps = [rnd.choice(laws3) for _ in range(n)]
        qs = [rnd.choice(laws3) for _ in range(n - 1)]
        tau = rnd.choice(TAUS)
        law = exact.window_law(ps, qs, tau)
        assert sum(law.values()) == 1
        alphas = [exact.acceptance_probability(ps[j], qs[j], tau) for j in range(n - 1)]
        for k in range(n):
            want = F(1)
            for a in alphas[:k]:
                want *= a
            got = sum(pr for (kk, _), pr in law.items() if kk >= k)
            assert got == want
        # token emitted at position i, given the window reached position i, is distributed as p_i
        for i in range(n):
            reach = sum(pr for (kk, _), pr in law.items() if kk >= i)
            if reach == 0:
                continue
            marg = [F(0)] * 3
            for (kk, toks), pr in law.items():
                if kk >= i:
                    marg[toks[i]] += pr
            assert [m / reach for m in marg] == ps[i]
