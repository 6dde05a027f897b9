"""Pins for the oracle's per-step thresholds and cumulative floor.

* The page's own numbers (regolith audit "rank-1 moce and step-aware
  speculative retention", section economics and confidence): with draft
  probabilities (0.5, 0.5, 0.5), a flat 0.35 gate keeps all three drafts, a
  cumulative floor of 0.2 keeps two, and the schedule (0.1, 0.35, 0.55) keeps
  two; a first probability of 0.2 fails the flat 0.35 gate but passes the
  cheap-first schedule. With p = q every offered draft is accepted, so the
  accept length counts the drafts the gates keep.
* Losslessness under both knobs, by exhaustive enumeration in exact
  arithmetic: for every accepted prefix that reaches position i, the token
  emitted at i is distributed exactly as p_i, although the gate depends on the
  prefix.
* The schedule's last threshold repeats (section schedule behavior), equality
  passes, and invalid knob values fail closed.
"""
import json
import os
import random
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact
from oracle import verify as ov

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _window(qd, V=2):
    """One request of len(qd) drafts plus a bonus row, p = q at every row, D = token 0.

    Row j's draft law puts probability qd[j] on token 0 and spreads the rest evenly.
    """
    n = len(qd) + 1
    tl = np.zeros((n, V))
    for j, a in enumerate(qd):
        rest = (1.0 - a) / (V - 1)
        tl[j] = np.log(np.array([a] + [rest] * (V - 1)))
    dl = tl.copy()
    dt = np.zeros(n, dtype=np.int64)
    dt[-1] = -1
    return tl, dl, dt


def _accept_len(qd, tau=0.0, steps=None, min_cum=0.0, seed=3):
    tl, dl, dt = _window(qd)
    st = None if steps is None else np.array(list(steps) + [0.0], dtype=np.float64)
    return ov.verify_request(tl, dl, dt, 1.0, tau, seed, 0, tau_steps=st, min_cum=min_cum)


def test_page_example_retention_counts():
    g = _gold("schedule_example.json")
    qd = g["draft_probs"]
    assert np.allclose(np.cumprod(qd), g["prefix_products"])
    r = g["retained"]
    assert _accept_len(qd, tau=r["flat"]["tau"]).accept_len == r["flat"]["count"]
    res = _accept_len(qd, min_cum=r["cumulative"]["min_cum"])
    assert res.accept_len == r["cumulative"]["count"]
    assert res.rows[-1].verdict == ov.NULL          # the failed gate ends the prefix
    assert _accept_len(qd, steps=r["schedule"]["steps"]).accept_len == r["schedule"]["count"]
    first = g["first_prob_0_2"]
    qd2 = [0.2, 0.5, 0.5]
    assert (_accept_len(qd2, tau=0.35).accept_len >= 1) == first["flat_0_35_retains_first"]
    assert (_accept_len(qd2, steps=r["schedule"]["steps"]).accept_len >= 1) == first["schedule_retains_first"]


def test_both_gates_compose_by_and():
    qd = [0.5, 0.5, 0.5]
    # schedule alone keeps 2, floor alone keeps 2; a floor of 0.3 alone keeps 1 (0.25 < 0.3)
    assert _accept_len(qd, min_cum=0.3).accept_len == 1
    assert _accept_len(qd, steps=[0.1, 0.35, 0.55], min_cum=0.3).accept_len == 1
    assert _accept_len(qd, steps=[0.1, 0.6, 0.1], min_cum=0.2).accept_len == 1
    # a floor of 0 turns the cumulative gate off
    assert _accept_len(qd, min_cum=0.0).accept_len == 3


def test_equality_passes_cumulative_gate():
    # products 0.5, 0.25: a floor of exactly 0.25 keeps the second draft (0.25 >= 0.25)
    qd = [0.5, 0.5, 0.5]
    assert _accept_len(qd, min_cum=0.25).accept_len == 2
    assert _accept_len(qd, min_cum=0.125).accept_len == 3


def test_step_thresholds_override_request_tau():
    qd = [0.5, 0.5, 0.5]
    assert _accept_len(qd, tau=0.9, steps=[0.1, 0.1, 0.1]).accept_len == 3
    assert _accept_len(qd, tau=0.0, steps=[0.1, 0.9, 0.1]).accept_len == 1


def test_invalid_knobs_fail_closed():
    qd = [0.5, 0.5, 0.5]
    for mc in (float("nan"), float("inf"), -0.1):
        assert _accept_len(qd, min_cum=mc).accept_len == -1
    # a NaN step threshold fails closed on a row that is tested ...
    assert _accept_len(qd, steps=[0.1, float("nan"), 0.1]).accept_len == -1
    # ... but not on a row behind the stop
    assert _accept_len(qd, steps=[0.9, float("nan"), 0.1]).accept_len == 0


TAUS = [F(0), F(1, 4), F(1, 3), F(1, 2), F(2, 3), F(1)]
FLOORS = [F(0), F(1, 10), F(1, 5), F(1, 3), F(1, 2), F(1)]


def test_lossless_under_schedule_and_floor_by_enumeration():
    laws = list(exact.all_rational_laws(3, 4))
    rnd = random.Random(11)
    checked = 0
    for _ in range(120):
        n = rnd.randint(2, 4)
        ps = [rnd.choice(laws) for _ in range(n)]
        qs = [rnd.choice(laws) for _ in range(n - 1)]
        steps = [rnd.choice(TAUS) for _ in range(n - 1)]
        floor = rnd.choice(FLOORS)
        law = exact.window_law(ps, qs, F(0), tau_steps=steps, min_cum=floor)
        assert sum(law.values()) == 1
        # for every accepted prefix that reaches position i, token i is distributed as p_i
        for i in range(n):
            by_prefix = {}
            for (k, toks), pr in law.items():
                if k >= i:
                    by_prefix.setdefault(toks[:i], [F(0)] * 3)[toks[i]] += pr
            for pre, w in by_prefix.items():
                tot = sum(w)
                assert [x / tot for x in w] == ps[i], (i, pre)
                checked += 1
    assert checked > 200


def test_floor_changes_acceptance_as_a_product_gate():
    # q puts 1/2 on each of two tokens; with p = q every offered draft is accepted.
    half = [F(1, 2), F(1, 2)]
    law = exact.window_law([half] * 4, [half] * 3, F(0), min_cum=F(1, 5))
    ks = {k for (k, _) in law}
    assert ks == {2}   # products 1/2, 1/4 pass the floor 1/5, 1/8 does not
    law = exact.window_law([half] * 4, [half] * 3, F(0), tau_steps=[F(1, 10), F(7, 20), F(11, 20)])
    assert {k for (k, _) in law} == {2}
