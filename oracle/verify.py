"""Plain fp64 CPU oracle of the speculative-decoding verify sampler.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.
The product path (the HIP library and its binding) never imports it.

The oracle follows the method's steps in order, one request and one row at a
time, in float64 on the exact input values. A bf16 or fp32 logit converts to
float64 without rounding. Citations name the page and the section:

* Strata PR #3416 "[Engine] Preserve target probabilities in gated MTP",
  section Approach. The retained measure mu = q * [q >= tau] is not
  renormalised. A failed gate makes an explicit NULL row. An offered token D
  is accepted with probability min(1, p(D)/mu(D)). Rejection and NULL both
  draw from the normalised positive part of p - mu. A row with no attempted
  proposal stays an ordinary target (bonus) sample.
* regolith audit "rank-1 moce and step-aware speculative retention",
  section schedule behavior. Equality passes the gate, and a failed gate ends
  the contiguous prefix. The same section describes two optional knobs,
  taken here as inputs: a per-step threshold that overrides the request's
  tau for its row, and a cumulative floor on the product of the draft
  probabilities of the drafted tokens so far, this row's included, computed
  in double and reset for every window. Both gates must pass. For row j the
  product condition q_0(D_0) ... q_j(D_j) >= min_cum is a threshold on
  q_j(D_j). Gating mu_j with that same threshold,
      tau_j = max(step threshold, min_cum / (q_0(D_0) ... q_{j-1}(D_{j-1}))),
  keeps the method lossless: tau_j depends only on the accepted prefix.
  A floor of 0 disables the cumulative gate.
* mlxcel PR #992, section What changed. The accept test compares a uniform
  against p and q in the form u*q(t) <= p(t) and requires p(t) > 0, so that a
  q that underflowed to zero cannot admit a token with p = 0. This oracle uses
  the strict form u*mu(D) < p(D), which carries that p > 0 requirement. See
  ``_accept``.
* mlxcel PR #992, section What changed. The sampler's filter chain
  (temperature, top-k, top-p, min-p) defines the effective p and q. The
  target's and the draft's filters are optional inputs per request. See
  ``filters`` for the readings and the flag F5.
* mlxcel PR #992, section Temperature 0. A greedy configuration turns p and q
  into one-hot argmax indicators, so no randomness decides anything.
* mlxcel PR #992, section Two metric corrections. A chain stops at its first
  rejection, and the positions behind it are never tested.

Readings where the pages leave a step open:

* p = softmax(target/T) and q = softmax(draft/T), at the request's own
  temperature T.
* The residual draw is an exponential race: token = argmax_x w[x] / E[x],
  with E[x] i.i.d. Exp(1) from Philox and ties going to the lower index. Its
  law is w / sum(w). mlxcel PR #992 (section What changed) draws the same law
  by Gumbel-max on log(w).
* A residual with zero total mass falls back to a race over p.
* draft_tokens[r] == -1, or any id outside [0, V), means "no proposal". Such a
  row, and the last row of every request, is a bonus row: one race over p.
* Temperature must be 0 or lie in [2**-14, 2**14]. tau must not be NaN, nor
  the step threshold of a row the method tests. The cumulative floor must be
  finite and >= 0.
  Logits must be finite or -inf. A row that contains NaN or +inf, or holds
  only -inf, is invalid, and so is its request. This is checked only on rows
  the method actually evaluates. An invalid request emits nothing: its
  accept length is -1 and all of its slots are -1.
* row_offsets must be strictly increasing from 0 to R. Otherwise every output
  is -1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import philox
from .filters import Filter, filter_active, filter_valid, filtered_distribution

# Row verdicts (also the codes the GPU side reports in its row diagnostics).
ACCEPT, REJECT, NULL, BONUS = 1, 2, 3, 4
VERDICT_NAMES = {0: "untested", ACCEPT: "accept", REJECT: "reject", NULL: "null", BONUS: "bonus"}

T_MIN = 2.0 ** -14
T_MAX = 2.0 ** 14
FLAG_EPS = 1e-6

# Flag bits (decision boundaries within FLAG_EPS; see ``verify_request``).
F_ACCEPT = 1      # F1: the accept uniform is near p(D)/mu(D)
F_GATE = 2        # F2: q(D) is near tau
F_RACE = 4        # F3: the two best race keys are near each other
F_SUPPORT = 8     # F4: some q_x is near tau, or the residual mass is near 0, in a residual race
F_FILTER = 16     # F5: a top-p or min-p decision of an evaluated row is near its boundary


# ---------------------------------------------------------------- decoding

def decode_logits(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of bf16 (uint16 bit patterns) or fp32 logits."""
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- the method's steps

def temperature_valid(T: float) -> bool:
    return T == 0.0 or (T_MIN <= T <= T_MAX)


def row_valid(logits: np.ndarray) -> bool:
    """Finite or -inf everywhere, and at least one finite entry."""
    if np.isnan(logits).any() or np.isposinf(logits).any():
        return False
    return bool(np.isfinite(logits).any())


def argmax_lowest(x: np.ndarray) -> int:
    """Index of the largest entry; ties go to the lowest index."""
    return int(np.argmax(x))


def softmax(logits: np.ndarray, T: float) -> np.ndarray:
    """softmax(logits / T) in float64, max-subtracted. -inf entries get probability 0."""
    z = logits / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def distribution(logits: np.ndarray, T: float) -> np.ndarray:
    """p (target) or q (draft) at temperature T. T == 0 gives the one-hot argmax indicator."""
    if T == 0.0:
        out = np.zeros_like(logits)
        out[argmax_lowest(logits)] = 1.0
        return out
    return softmax(logits, T)


def row_distribution(logits: np.ndarray, T: float, filt: Filter | None):
    """(p, near): ``distribution`` with the sampler's filter chain applied when T > 0.

    The filters follow mlxcel PR #992, section What changed (see ``filters``).
    ``near`` flags a filter decision within its band.
    """
    if T > 0.0 and filt is not None and filter_active(filt, logits.size):
        return filtered_distribution(logits, T, filt)
    return distribution(logits, T), False


def retained_measure(q: np.ndarray, tau: float) -> np.ndarray:
    """mu = q * [q >= tau], left unnormalised (Strata PR #3416, Approach)."""
    return np.where(q >= tau, q, 0.0)


def race(w: np.ndarray, E: np.ndarray) -> int:
    """Exponential race: argmax_x w[x]/E[x], ties to the lower index. Law: w / sum(w)."""
    return argmax_lowest(w / E)


def _accept(u: float, mu_D: float, p_D: float) -> bool:
    """Accept iff u*mu(D) < p(D). With u uniform on [0, 1) this has probability min(1, p/mu)."""
    return u * mu_D < p_D


# ---------------------------------------------------------------- one request

@dataclass
class RowRecord:
    j: int
    verdict: int
    p_D: float = float("nan")
    q_D: float = float("nan")
    mu_D: float = float("nan")
    u: float = float("nan")
    resid_mass: float = float("nan")


@dataclass
class RequestResult:
    tokens: list            # emitted tokens: k accepted drafts, then one residual/bonus token
    accept_len: int         # k, or -1 for an invalid request
    rows: list = field(default_factory=list)   # RowRecord per evaluated row
    flags: int = 0          # OR of the F_* bits over evaluated rows


def _top2_gap(keys: np.ndarray, cond: np.ndarray | None):
    """Relative gap between the two largest keys and the larger of their sensitivity factors."""
    if keys.size < 2:
        return np.inf, 1.0
    i2 = np.argpartition(-keys, 1)[:2]
    a, b = (i2[0], i2[1]) if keys[i2[0]] >= keys[i2[1]] else (i2[1], i2[0])
    k1, k2 = keys[a], keys[b]
    if k1 <= 0.0:
        return np.inf, 1.0
    c = 1.0 if cond is None else max(cond[a], cond[b], 1.0)
    return (k1 - k2) / k1, c


def sampler_match_request(tl: np.ndarray, dt: np.ndarray, T: float, seed: int, b: int) -> RequestResult:
    """The sampler-match rule (mlxcel PR #992, section The premise correction).

    Every tested row takes a fresh draw t from the target p, here the row's
    exponential race over p (the same random numbers as the method's race on
    that row). The drafted token is accepted iff it equals t, and t is emitted
    on both branches, so every emitted token is a draw from p. The rule reads
    neither q nor a gate. Its acceptance is sum_x p(x) q(x) for D ~ q (the
    same page, section The acceptance ceiling). At T = 0 the draw is the
    lowest-index argmax. The last row, or a row with no proposal, is a bonus
    draw as in the method.

    Flags: F3 when a race's two best keys p/E lie within a relative FLAG_EPS.
    """
    n, V = tl.shape
    res = RequestResult(tokens=[], accept_len=-1)
    if not temperature_valid(T):
        return res
    for j in range(n):
        if not row_valid(tl[j]):
            res.tokens = []
            res.rows.append(RowRecord(j=j, verdict=0))
            return res
        p = distribution(tl[j], T)
        if T > 0.0:
            E = philox.race_exponentials(seed, b, j, V)
            t = race(p, E)
            gap, _ = _top2_gap(p / E, None)
            if gap < FLAG_EPS:
                res.flags |= F_RACE
        else:
            t = argmax_lowest(p)
        D = int(dt[j])
        bonus = (j == n - 1) or not (0 <= D < V)
        if not bonus and D == t:
            res.rows.append(RowRecord(j=j, verdict=ACCEPT, p_D=float(p[D])))
            res.tokens.append(D)
            continue
        res.rows.append(RowRecord(j=j, verdict=BONUS if bonus else REJECT))
        res.tokens.append(t)
        res.accept_len = len(res.tokens) - 1
        return res
    raise AssertionError("unreachable: the last row is always a bonus row")


def verify_request(tl: np.ndarray, dl: np.ndarray, dt: np.ndarray, T: float, tau: float,
                   seed: int, b: int, rule: str = "mu", tau_steps: np.ndarray | None = None,
                   min_cum: float = 0.0, tfilt: Filter | None = None,
                   dfilt: Filter | None = None) -> RequestResult:
    """Verify one request's window of rows.

    ``tl``, ``dl`` are float64 [n, V] target and draft logits, and ``dt`` is
    [n] draft tokens. Row n-1 is the bonus row. ``b`` is the request's index
    in the batch, which keys its random stream.

    ``tau_steps`` ([n], optional) holds each row's step threshold, which
    replaces ``tau`` for that row. ``min_cum`` is the cumulative floor (0 turns
    that gate off). Row j gates at tau_j = max(step threshold, min_cum / the
    product of q_i(D_i) over the accepted rows i < j).

    ``tfilt`` and ``dfilt`` are the target's and the draft's filter chains
    (top-k, top-p, min-p; mlxcel PR #992, section What changed). When T > 0,
    p and q are the filtered distributions, and an invalid filter makes the
    request invalid. A greedy request ignores both.

    ``rule`` selects the method ("mu") or a deliberately wrong rule that the
    pages use as a negative control:

    * "original": the biased gated verifier of Strata PR #3416, section
      Problem and result. It accepts with min(1, p/q) using the unfiltered q,
      draws from (p - q)+ on rejection, and turns a failed gate into a plain
      target sample.
    * "resample_p": mu acceptance, but a rejection resamples from p instead of
      the residual. This is the naive mistake in mlxcel PR #992, section
      The distributional argument.
    * "argmax": argmax-against-argmax. D is accepted iff it is the target's
      argmax, and a rejection emits that argmax (mlxcel PR #992, section The
      acceptance ceiling).

    ``rule="sampler_match"`` runs ``sampler_match_request``: a correct rule
    with a lower acceptance, which the pages compare the method against. It
    ignores the draft logits, tau, the schedule and the filters.

    Flags (method only, T > 0) mark requests whose result is decided within
    FLAG_EPS of a boundary, where float32 arithmetic may legitimately decide
    the other way:

    * F1: an offered row with |u - p(D)/mu(D)| < eps.
    * F2: tau_j > 0 and |q(D) - tau_j| < eps.
    * F3: a race whose two best keys k1 >= k2 have (k1 - k2)/k1 < eps * c.
      Here c = max(1, (p+mu)/r) over the two tokens of a residual race with
      r = p - mu. That is the factor by which a relative error of eps in p
      and mu moves the key r/E.
    * F4: a residual race with some |q_x - tau_j| < eps (tau_j > 0), or a
      residual mass below eps.
    * F5: a filter decision near its boundary on a row the method evaluates
      (``filters.threshold``).
    """
    if rule == "sampler_match":
        return sampler_match_request(tl, dt, T, seed, b)
    n, V = tl.shape
    res = RequestResult(tokens=[], accept_len=-1)
    if not temperature_valid(T) or np.isnan(tau) or not (np.isfinite(min_cum) and min_cum >= 0.0):
        return res
    if T > 0.0 and any(f is not None and not filter_valid(f) for f in (tfilt, dfilt)):
        return res
    cum = 1.0  # product of q_i(D_i) over the accepted rows so far
    for j in range(n):
        D = int(dt[j])
        bonus = (j == n - 1) or not (0 <= D < V)
        if not row_valid(tl[j]):
            res.tokens = []
            res.rows.append(RowRecord(j=j, verdict=0))
            return res
        p, near = row_distribution(tl[j], T, tfilt)
        if near and rule == "mu":
            res.flags |= F_FILTER
        if bonus:
            E = philox.race_exponentials(seed, b, j, V)
            tok = race(p, E)
            if T > 0.0:
                gap, _ = _top2_gap(p / E, None)
                if gap < FLAG_EPS:
                    res.flags |= F_RACE
            res.tokens.append(tok)
            res.rows.append(RowRecord(j=j, verdict=BONUS))
            res.accept_len = len(res.tokens) - 1
            return res
        if not row_valid(dl[j]):
            res.tokens = []
            res.rows.append(RowRecord(j=j, verdict=0))
            return res
        q, near = row_distribution(dl[j], T, dfilt)
        if near and rule == "mu":
            res.flags |= F_FILTER
        rec = RowRecord(j=j, verdict=0, p_D=float(p[D]), q_D=float(q[D]))
        tau_j = tau if tau_steps is None else float(tau_steps[j])
        if np.isnan(tau_j):
            res.tokens = []
            res.rows.append(RowRecord(j=j, verdict=0))
            return res
        if min_cum > 0.0:
            tau_j = max(tau_j, min_cum / cum)

        if rule == "argmax":
            am = argmax_lowest(p)
            if D == am:
                rec.verdict = ACCEPT
                res.rows.append(rec)
                res.tokens.append(D)
                continue
            rec.verdict = REJECT
            res.rows.append(rec)
            res.tokens.append(am)
            res.accept_len = len(res.tokens) - 1
            return res

        mu = retained_measure(q, tau_j)
        offered = q[D] >= tau_j
        if rule == "mu" and T > 0.0 and tau_j > 0.0 and abs(q[D] - tau_j) < FLAG_EPS:
            res.flags |= F_GATE
        if offered:
            mu_D = q[D] if rule == "original" else mu[D]
            rec.mu_D = float(mu_D)
            # At T == 0, p(D) is 0 or 1 and mu(D) <= 1, so u*mu(D) < p(D) has the
            # same outcome for every u in [0, 1): no uniform is drawn.
            u = philox.accept_uniform(seed, b, j) if T > 0.0 else 0.0
            rec.u = u if T > 0.0 else float("nan")
            if rule == "mu" and T > 0.0 and mu_D > 0.0 and abs(u - p[D] / mu_D) < FLAG_EPS:
                res.flags |= F_ACCEPT
            if _accept(u, mu_D, p[D]):
                rec.verdict = ACCEPT
                res.rows.append(rec)
                res.tokens.append(D)
                cum *= q[D]
                continue
            rec.verdict = REJECT
        else:
            rec.verdict = NULL
            rec.mu_D = 0.0

        # Rejection or NULL: draw from the normalised positive part of p - mu.
        if rule == "original":
            w = np.maximum(p - q, 0.0) if offered else p
        elif rule == "resample_p":
            w = p
        else:
            w = np.maximum(p - mu, 0.0)
        R = float(w.sum())
        rec.resid_mass = R
        E = philox.race_exponentials(seed, b, j, V)
        if R > 0.0:
            tok = race(w, E)
        else:
            tok = race(p, E)
        if rule == "mu" and T > 0.0:
            if R > 0.0:
                with np.errstate(divide="ignore", invalid="ignore"):
                    cond = np.where(w > 0.0, (p + mu) / np.where(w > 0.0, w, 1.0), 1.0)
                gap, c = _top2_gap(w / E, cond)
            else:
                gap, c = _top2_gap(p / E, None)
            if gap < FLAG_EPS * c:
                res.flags |= F_RACE
            if R < FLAG_EPS or (tau_j > 0.0 and bool((np.abs(q - tau_j) < FLAG_EPS).any())):
                res.flags |= F_SUPPORT
        res.rows.append(rec)
        res.tokens.append(tok)
        res.accept_len = len(res.tokens) - 1
        return res
    raise AssertionError("unreachable: the last row is always a bonus row")


# ---------------------------------------------------------------- a batch

def row_offsets_valid(ro: np.ndarray, R: int) -> bool:
    ro = np.asarray(ro, dtype=np.int64)
    if ro.size < 1 or ro[0] != 0 or ro[-1] != R:
        return False
    return bool(np.all(np.diff(ro) > 0))


@dataclass
class BatchResult:
    out_tokens: np.ndarray      # [R] int32
    out_accept_len: np.ndarray  # [B] int32
    flags: np.ndarray           # [B] int32, F_* bits
    verdict: np.ndarray         # [R] int32 (0 = row not tested)
    p_D: np.ndarray             # [R] float64 (nan where not defined)
    q_D: np.ndarray
    mu_D: np.ndarray
    u: np.ndarray
    resid_mass: np.ndarray      # [R] float64, set on residual rows only


def request_filter(triple, b: int) -> Filter | None:
    """Request b's filter from a (top_k, top_p, min_p) triple of [B] arrays (None: off)."""
    if triple is None:
        return None
    k, tp, mp = triple
    return Filter(top_k=0 if k is None else int(np.asarray(k, dtype=np.int32)[b]),
                  top_p=1.0 if tp is None else float(np.asarray(tp, dtype=np.float32)[b]),
                  min_p=0.0 if mp is None else float(np.asarray(mp, dtype=np.float32)[b]))


def verify_batch(target, draft, draft_tokens, row_offsets, temperature, tau, seed: int,
                 dtype: str, requests=None, rule: str = "mu", tau_step=None, min_cum=None,
                 target_filter=None, draft_filter=None) -> BatchResult:
    """Verify every request of a batch (or only those listed in ``requests``).

    ``target`` and ``draft`` are [R, V] arrays of bf16 bit patterns (uint16) or
    fp32 values. The other arguments mirror the C-ABI entry point. Requests not
    in ``requests`` keep -1 outputs. ``tau_step`` ([R] float32) and ``min_cum``
    ([B] float32) are the optional per-row step thresholds and per-request
    cumulative floors. ``target_filter`` and ``draft_filter`` are optional
    triples (top_k [B] int32, top_p [B] float32, min_p [B] float32), any
    member of which may be None (that filter off).
    """
    target = np.asarray(target)
    R, V = target.shape
    ro = np.asarray(row_offsets, dtype=np.int64)
    B = ro.size - 1
    out_tokens = np.full(R, -1, dtype=np.int32)
    out_len = np.full(B, -1, dtype=np.int32)
    flags = np.zeros(B, dtype=np.int32)
    verdict = np.zeros(R, dtype=np.int32)
    nan = lambda: np.full(R, np.nan)  # noqa: E731
    p_D, q_D, mu_D, u, rm = nan(), nan(), nan(), nan(), nan()
    if not row_offsets_valid(ro, R):
        return BatchResult(out_tokens, out_len, flags, verdict, p_D, q_D, mu_D, u, rm)
    temperature = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    tau = np.asarray(tau, dtype=np.float32).astype(np.float64)
    dt = np.asarray(draft_tokens, dtype=np.int64)
    ts = None if tau_step is None else np.asarray(tau_step, dtype=np.float32).astype(np.float64)
    mc = None if min_cum is None else np.asarray(min_cum, dtype=np.float32).astype(np.float64)
    todo = range(B) if requests is None else requests
    for b in todo:
        lo, hi = int(ro[b]), int(ro[b + 1])
        tl = decode_logits(target[lo:hi], dtype)
        dl = decode_logits(np.asarray(draft)[lo:hi], dtype)
        rr = verify_request(tl, dl, dt[lo:hi], float(temperature[b]), float(tau[b]), seed, b, rule,
                            None if ts is None else ts[lo:hi], 0.0 if mc is None else float(mc[b]),
                            request_filter(target_filter, b), request_filter(draft_filter, b))
        flags[b] = rr.flags
        for rec in rr.rows:
            r = lo + rec.j
            verdict[r] = rec.verdict
            p_D[r], q_D[r], mu_D[r], u[r], rm[r] = rec.p_D, rec.q_D, rec.mu_D, rec.u, rec.resid_mass
        if rr.accept_len < 0:
            continue
        out_len[b] = rr.accept_len
        out_tokens[lo:lo + len(rr.tokens)] = rr.tokens
    return BatchResult(out_tokens, out_len, flags, verdict, p_D, q_D, mu_D, u, rm)


# ---------------------------------------------------------------- closed forms

def acceptance_probability(p: np.ndarray, mu: np.ndarray) -> float:
    """P(accept) of one offered-or-NULL row with D ~ q: sum_x min(p(x), mu(x)).

    Ungated (mu = q) this is the maximal-coupling ceiling 1 - TV(p, q)
    (mlxcel PR #992, section The acceptance ceiling).
    """
    return float(np.minimum(p, mu).sum())


def sum_prod(p: np.ndarray, q: np.ndarray) -> float:
    """sum_x p(x) q(x): acceptance of the sampler-match rule (mlxcel PR #992, The acceptance ceiling)."""
    return float((p * q).sum())


def row_sums(target, draft, draft_tokens, row_offsets, temperature, tau, dtype: str,
             tau_step=None, min_cum=None, target_filter=None, draft_filter=None):
    """Per proposal row: sum_x min(p(x), mu(x)) and sum_x p(x) q(x).

    The first is the probability that the row accepts its draft given that its
    prefix was accepted (Strata PR #3416, section Approach; mlxcel PR #992,
    section The acceptance ceiling); the second is the sampler-match rule's.
    mu uses the row's gate threshold: its step threshold (tau[b] without one),
    raised by the cumulative floor over the drafted tokens before it, as in
    ``verify_request``. Proposal rows are the rows before a request's first
    row without a proposal and before its last row; every other row gets NaN.
    A request that ``verify_request`` would fail closed on its knobs, or a row
    whose logits are invalid, gets NaN.

    With ``target_filter`` / ``draft_filter`` (triples as in ``verify_batch``),
    p and q are the filtered distributions (mlxcel PR #992, section What
    changed), and a request whose filter values are invalid at T > 0 gets NaN.

    Returns (sum_min, sum_pq, near_gate): near_gate[r] marks a row with some
    |q(x) - tau_j| < FLAG_EPS (tau_j > 0), or a filter decision in its flag
    band, where float arithmetic may legitimately decide the other way.
    """
    target = np.asarray(target)
    R, V = target.shape
    ro = np.asarray(row_offsets, dtype=np.int64)
    B = ro.size - 1
    smin = np.full(R, np.nan)
    spq = np.full(R, np.nan)
    near = np.zeros(R, dtype=bool)
    if not row_offsets_valid(ro, R):
        return smin, spq, near
    temperature = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    tau = np.asarray(tau, dtype=np.float32).astype(np.float64)
    dt = np.asarray(draft_tokens, dtype=np.int64)
    ts = None if tau_step is None else np.asarray(tau_step, dtype=np.float32).astype(np.float64)
    mc = None if min_cum is None else np.asarray(min_cum, dtype=np.float32).astype(np.float64)
    for b in range(B):
        lo, hi = int(ro[b]), int(ro[b + 1])
        T = float(temperature[b])
        floor = 0.0 if mc is None else float(mc[b])
        if not temperature_valid(T) or np.isnan(tau[b]) or not (np.isfinite(floor) and floor >= 0.0):
            continue
        tf, df = request_filter(target_filter, b), request_filter(draft_filter, b)
        if T > 0.0 and any(f is not None and not filter_valid(f) for f in (tf, df)):
            continue
        cum = 1.0
        for j in range(hi - lo - 1):
            r = lo + j
            D = int(dt[r])
            if not 0 <= D < V:
                break
            tl = decode_logits(target[r:r + 1], dtype)[0]
            dl = decode_logits(np.asarray(draft)[r:r + 1], dtype)[0]
            if not (row_valid(tl) and row_valid(dl)):
                break
            p, near_p = row_distribution(tl, T, tf)
            q, near_q = row_distribution(dl, T, df)
            tau_j = float(tau[b]) if ts is None else float(ts[r])
            if np.isnan(tau_j):
                break
            if floor > 0.0:
                tau_j = max(tau_j, floor / cum)
            smin[r] = acceptance_probability(p, retained_measure(q, tau_j))
            spq[r] = sum_prod(p, q)
            near[r] = near_p or near_q or (tau_j > 0.0 and bool((np.abs(q - tau_j) < FLAG_EPS).any()))
            cum *= q[D]
    return smin, spq, near
