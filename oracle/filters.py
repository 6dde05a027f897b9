"""Plain fp64 oracle of the sampler's filter chain: top-k, top-p, min-p.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.

mlxcel PR #992, section What changed: the sampler scales the logits by the
temperature, then applies top-k, then top-p, then min-p, and the effective
distribution is the softmax of what is left (zero elsewhere). The verify
sampler's p and q are these filtered distributions, each with its own
filter parameters. The same section notes that a greedy configuration
(temperature 0 or top_k 1) gives the one-hot argmax indicator. The page's
tests (section Where chi-square is blind) require that no token outside a
filtered target's support is ever emitted.

Readings where the page leaves a step open:

* Every filter keeps the tokens whose logit reaches a threshold, and ties at
  the threshold are all kept. Since T > 0, ordering by logit and by
  logit / T is the same, so the thresholds are taken on the raw logits. With
  a unique maximum, top_k = 1 keeps just the argmax (the page's one-hot);
  with a tied maximum it keeps every tied token.
* top-k (k > 0 and k < V): the threshold is the k-th largest logit, counted
  with multiplicity. k = 0, or k >= V, turns it off. A negative k is invalid.
* top-p (0 < top_p < 1) works on the distribution that top-k leaves,
  renormalised. It keeps the fewest largest tokens whose mass reaches top_p,
  and the token whose mass crosses top_p is kept. Its threshold is the
  largest logit v with C(v) >= top_p * S1, where C(v) is the mass of the
  tokens with logit >= v and S1 the mass of top-k's set. top_p >= 1 turns it
  off; NaN or top_p <= 0 is invalid.
* min-p (0 < min_p <= 1) keeps the tokens whose probability is at least
  min_p times the largest. In log form that is (x - m) / T >= ln(min_p),
  where m is the row maximum, and this oracle tests it in that form. The
  ratio does not change under renormalisation, and the maximum survives
  every filter, so the earlier filters do not move it. min_p = 0 turns it
  off; NaN, min_p < 0 or min_p > 1 is invalid.
* The kept set is the tokens at or above the largest of the three
  thresholds. p is the fp64 softmax over the kept set at temperature T.
* A greedy request (T = 0) ignores its filters: it is already the one-hot
  argmax, and its filter values are not checked.

Decisions within a band of a boundary are flagged. There the float
arithmetic of another implementation may decide the other way:

* top-p: C(v) within FILTER_EPS * S1 + TAIL_EPS * (S1 - C(theta_p)) of
  top_p * S1, either at the crossing value or at the next larger value (if any). The
  second term allows for an implementation that sums the mass below the
  kept set in float32: S1 includes that mass when top-k is off, and a
  float32 exp2 term with |log2 e| <= 80 carries a relative error below 1e-5.
* min-p: some logit with |(x - m)/T - ln(min_p)| <= MINP_EPS * max(1, |ln(min_p)|),
  for min_p < 1 (min_p = 1 keeps exactly the logits equal to m).
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

FILTER_EPS = 1e-9
TAIL_EPS = 1e-5
MINP_EPS = 1e-12


@dataclass(frozen=True)
class Filter:
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0


NO_FILTER = Filter()


def filter_valid(f: Filter) -> bool:
    """Parameter ranges (readings above). Checked for requests with T > 0 only."""
    if f.top_k < 0:
        return False
    if math.isnan(f.top_p) or f.top_p <= 0.0:
        return False
    if math.isnan(f.min_p) or f.min_p < 0.0 or f.min_p > 1.0:
        return False
    return True


def filter_active(f: Filter, V: int) -> bool:
    return (0 < f.top_k < V) or f.top_p < 1.0 or f.min_p > 0.0


def threshold(x: np.ndarray, T: float, f: Filter):
    """Keep-threshold of one row: (theta, near).

    ``x`` holds the row's exact logits in float64 (finite or -inf, with at least
    one finite entry), and T > 0. The kept tokens are those with x >= theta.
    theta is -inf when no filter is active. ``near`` is True when a top-p or
    min-p decision falls within its flag band.
    """
    V = x.size
    m = float(x.max())
    xs = -np.sort(-x)  # logits in decreasing order
    near = False

    theta_k = -np.inf
    if 0 < f.top_k < V:
        theta_k = float(xs[f.top_k - 1])

    theta_p = -np.inf
    if f.top_p < 1.0:
        e = np.exp((xs - m) / T)
        n_k = int(np.count_nonzero(xs >= theta_k))  # top-k's set is a prefix of xs
        cum = np.cumsum(e[:n_k])
        S1 = float(cum[-1])
        target = f.top_p * S1
        i = int(np.argmax(cum >= target))  # first position whose prefix mass reaches top_p
        v = xs[i]
        first = int(np.argmax(xs == v))
        last = n_k - 1 - int(np.argmax(xs[:n_k][::-1] == v))
        c_at = float(cum[last])                           # C(v)
        c_above = float(cum[first - 1]) if first > 0 else 0.0  # C at the next larger value
        band = FILTER_EPS * S1 + TAIL_EPS * max(S1 - c_at, 0.0)
        # At the largest value there is no larger one, so C(v) >= top_p * S1 is the only decision.
        if c_at - target <= band or (first > 0 and target - c_above <= band):
            near = True
        theta_p = float(v)

    theta_m = -np.inf
    if f.min_p > 0.0:
        lm = math.log(f.min_p)
        z = (xs - m) / T
        ok = z >= lm
        theta_m = float(xs[ok].min())
        band = MINP_EPS * max(1.0, abs(lm))
        # min_p = 1: ln(1) = 0 in every implementation, and (x - m)/T = 0 exactly iff x = m,
        # so the decision is exact.
        if lm != 0.0 and bool((np.abs(z[np.isfinite(z)] - lm) <= band).any()):
            near = True

    return max(theta_k, theta_p, theta_m), near


def filtered_distribution(x: np.ndarray, T: float, f: Filter | None):
    """(p, near): softmax(x / T) over the tokens the chain keeps, 0 elsewhere (T > 0)."""
    z = (x - x.max()) / T
    e = np.exp(z)
    near = False
    if f is not None and filter_active(f, x.size):
        theta, near = threshold(x, T, f)
        e = np.where(x >= theta, e, 0.0)
    return e / e.sum(), near
