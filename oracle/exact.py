"""Exact (rational) law of what the verify sampler emits, by enumeration.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.

Here p and q are given directly as lists of ``fractions.Fraction`` rather
than as logits. The drafted token D is marginalised over q. The accept
probability and the residual are used as exact numbers in place of random
draws. The result is the exact probability of each emitted sequence, so
losslessness ("the emitted token is distributed as p") can be checked with no
statistical slack.

The steps follow Strata PR #3416 "[Engine] Preserve target probabilities in
gated MTP", section Approach:

* mu = q * [q >= tau], not renormalised;
* an offered D is accepted with probability min(1, p(D)/mu(D));
* rejection and NULL draw from the normalised (p - mu)+;
* the last row is a bonus sample from p.

The "sampler_match" rule is the comparison rule of mlxcel PR #992, section
The premise correction: D is accepted iff it equals a fresh draw from p, and
that draw is emitted either way.

The "original" rule is that page's biased verifier from section Problem and
result. It accepts with min(1, p/q) using the unfiltered q and draws from
(p - q)+ on rejection. A failed gate becomes a plain sample from p.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import product


def _normalise(w):
    s = sum(w)
    return [x / s for x in w]


def retained_measure(q, tau):
    return [qi if qi >= tau else Fraction(0) for qi in q]


def residual_law(p, mu):
    """Normalised (p - mu)+. A residual with zero mass falls back to p (a reading)."""
    r = [max(pi - mi, Fraction(0)) for pi, mi in zip(p, mu)]
    if sum(r) == 0:
        return list(p)
    return _normalise(r)


def row_law(p, q, tau, rule="mu"):
    """Law of one proposal row with D ~ q.

    Returns (accepted, fallback). ``accepted[x]`` is P(D = x and D is
    accepted). ``fallback[x]`` is P(the row stops and emits x).
    """
    V = len(p)
    accepted = [Fraction(0)] * V
    fallback = [Fraction(0)] * V
    if rule == "sampler_match":
        # D ~ q and an independent fresh draw t ~ p; D is accepted iff D == t, and t is
        # emitted either way (mlxcel PR #992, section The premise correction).
        for x in range(V):
            accepted[x] = q[x] * p[x]
            fallback[x] = p[x] * (1 - q[x])
        return accepted, fallback
    mu = retained_measure(q, tau)
    for D in range(V):
        if q[D] == 0:
            continue
        if q[D] >= tau:                       # offered
            m = q[D] if rule == "original" else mu[D]
            a = min(Fraction(1), p[D] / m)
            accepted[D] += q[D] * a
            stop = q[D] * (1 - a)
            if rule == "original":
                law = residual_law(p, q)
            else:
                law = residual_law(p, mu)
        else:                                 # NULL (method) or plain target sample (original)
            stop = q[D]
            law = list(p) if rule == "original" else residual_law(p, mu)
        for x in range(V):
            fallback[x] += stop * law[x]
    return accepted, fallback


def first_token_distribution(p, q, tau, rule="mu"):
    """Law of the first emitted token of a one-draft window (row 0 proposes, row 1 is the bonus)."""
    accepted, fallback = row_law(p, q, tau, rule)
    return [a + f for a, f in zip(accepted, fallback)]


def acceptance_probability(p, q, tau):
    """sum_x min(p(x), mu(x)): the probability that the row accepts its draft."""
    mu = retained_measure(q, tau)
    return sum(min(a, b) for a, b in zip(p, mu))


def window_law(ps, qs, tau, rule="mu", tau_steps=None, min_cum=Fraction(0)):
    """Exact law of (accept_len, emitted tokens) for a window of n rows.

    ``ps`` has n target laws (row n-1 is the bonus row). ``qs`` has n-1 draft
    laws, one per proposal row. Rows are verified in order, and the first
    row that does not accept ends the window. Returns {(k, tokens): prob}.

    ``tau_steps`` (n-1 thresholds) replaces ``tau`` row by row, and a positive
    ``min_cum`` adds the cumulative gate: row j gates at
    max(step threshold, min_cum / prod_{i<j} q_i(D_i)) over the accepted prefix
    (regolith audit, section schedule behavior).
    """
    n = len(ps)
    assert len(qs) == n - 1
    out = {}

    def walk(j, prefix, prob, cum=Fraction(1)):
        if prob == 0:
            return
        if j == n - 1:
            for x, px in enumerate(ps[j]):
                if px:
                    key = (j, tuple(prefix) + (x,))
                    out[key] = out.get(key, Fraction(0)) + prob * px
            return
        tau_j = tau if tau_steps is None else tau_steps[j]
        if min_cum > 0:
            tau_j = max(tau_j, min_cum / cum)
        accepted, fallback = row_law(ps[j], qs[j], tau_j, rule)
        for x, fx in enumerate(fallback):
            if fx:
                key = (j, tuple(prefix) + (x,))
                out[key] = out.get(key, Fraction(0)) + prob * fx
        for D, aD in enumerate(accepted):
            walk(j + 1, prefix + [D], prob * aD, cum * qs[j][D])

    walk(0, [], Fraction(1))
    return out


def all_rational_laws(V, denom):
    """Every probability vector of length V whose entries are multiples of 1/denom."""
    for parts in product(range(denom + 1), repeat=V - 1):
        s = sum(parts)
        if s <= denom:
            yield [Fraction(k, denom) for k in parts] + [Fraction(denom - s, denom)]
