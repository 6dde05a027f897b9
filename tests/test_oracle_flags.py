"""Pins for the oracle's decision-boundary flags F1 to F4.

The flags mark requests whose outcome is decided so close to a boundary that
float32 arithmetic may decide it the other way. Every GPU parity test leaves
flagged requests out of its bit-exact comparison, so a band that is too wide
would hide mismatches, and one that is too narrow would fail good kernels.

Each case is built from float32 logits and tuned, one float32 step at a time,
until the quantity the flag watches lies in a chosen window. The window is
computed here from the inputs in fp64, independently of the oracle's own
flag code. Each flag gets a case just inside its band and one just outside,
on both sides of the boundary where the boundary has two sides:

* F1, the accept test u*mu(D) < p(D) of Strata PR #3416 (section Approach) and
  mlxcel PR #992 (section What changed): |u - p(D)/mu(D)| against 1e-6.
* F2, the gate q(D) >= tau (Strata PR #3416, section Approach): |q(D) - tau|
  against 1e-6.
* F3, the exponential race: the relative gap of the two best keys against
  1e-6 * c, with c = max(1, (p + mu)/r) over the two tokens of a residual
  race (r = p - mu), and c = 1 for a race over p. A residual case whose gap
  lies between 1e-6 and 1e-6 * c pins the factor.
* F4, the residual's support: some q_x within 1e-6 of tau, or a residual mass
  below 1e-6.

A greedy request (T = 0) draws nothing and is never flagged.
"""
import numpy as np
import pytest

from oracle import philox
from oracle.verify import F_ACCEPT, F_GATE, F_RACE, F_SUPPORT, verify_request

BAND = 1e-6
INSIDE = (0.80 * BAND, 0.95 * BAND)
OUTSIDE = (1.05 * BAND, 1.25 * BAND)


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _softmax64(l):
    l = np.asarray(l, dtype=np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def _tune(measure, lo_x, hi_x, window):
    """A float32 knob x with measure(x) in window. measure must be non-decreasing in x.

    Bisection on x in fp64 finds the window's middle; the float32 values near it are then
    tried in turn, since measure only sees x rounded to float32.
    """
    target = 0.5 * (window[0] + window[1])
    a, b = float(lo_x), float(hi_x)
    assert measure(a) < target < measure(b), (measure(a), target, measure(b))
    for _ in range(200):
        m = 0.5 * (a + b)
        if measure(m) < target:
            a = m
        else:
            b = m
    x = np.float32(0.5 * (a + b))
    up, down = x, x
    for _ in range(400):
        for cand in (up, down):
            v = measure(float(cand))
            if window[0] <= v <= window[1]:
                return float(cand), v
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
    raise AssertionError(f"no float32 knob puts the measure in {window}")


def _flags(tl, dl, dt, tau, seed, b=0, T=1.0):
    return verify_request(_f32(tl), _f32(dl), np.asarray(dt, dtype=np.int64), T, float(np.float32(tau)),
                          seed, b).flags


def _seed_with_uniform(lo, hi, b=0, j=0):
    for seed in range(1000):
        if lo < philox.accept_uniform(seed, b, j) < hi:
            return seed
    raise AssertionError("no seed")


# ---------------------------------------------------------------- F1

@pytest.mark.parametrize("window,sign,fires", [(INSIDE, 1, True), (INSIDE, -1, True),
                                              (OUTSIDE, 1, False), (OUTSIDE, -1, False),
                                              ((0.0, 0.1 * BAND), 1, True)])
def test_f1_accept_band(window, sign, fires):
    # V = 2, tau = 0: q = (1/2, 1/2) = mu, p(0) = logistic(t). Row 0 offers D = 0; row 1 is the bonus.
    seed = _seed_with_uniform(0.3, 0.7)
    u = philox.accept_uniform(seed, 0, 0)

    def margin(t):  # sign * (p(D)/mu(D) - u), from the float32 logit
        pD = _softmax64(_f32([t, 0.0]))[0]
        return sign * (pD / 0.5 - u)

    x, m = _tune(lambda v: margin(sign * v), -3.0, 3.0, window)  # increasing in v
    t = sign * x
    assert window[0] <= margin(t) <= window[1]
    tl = [[t, 0.0], [4.0, -4.0]]
    dl = [[0.0, 0.0], [0.0, 0.0]]
    f = _flags(tl, dl, [0, -1], 0.0, seed)
    assert bool(f & F_ACCEPT) == fires, (m, f)


# ---------------------------------------------------------------- F2

@pytest.mark.parametrize("window,sign,fires", [(INSIDE, 1, True), (INSIDE, -1, True),
                                              (OUTSIDE, 1, False), (OUTSIDE, -1, False)])
def test_f2_gate_band(window, sign, fires):
    # V = 2: q(0) = logistic(s) near tau = 0.3; p = (1/2, 1/2), so an offered D is always
    # accepted (p/mu > 1.6) and F1 stays silent.
    tau = float(np.float32(0.3))

    def margin(s):  # sign * (q(D) - tau)
        return sign * (_softmax64(_f32([s, 0.0]))[0] - tau)

    x, m = _tune(lambda v: margin(sign * v), -3.0, 3.0, window)
    s = sign * x
    tl = [[0.0, 0.0], [4.0, -4.0]]
    dl = [[s, 0.0], [0.0, 0.0]]
    f = _flags(tl, dl, [0, -1], tau, seed=1)
    assert bool(f & F_GATE) == fires, (m, f)


def test_f2_needs_a_gate():
    # tau = 0 gates nothing, so q(D) near 0 cannot flag.
    f = _flags([[0.0, 0.0], [1.0, 0.0]], [[-30.0, 0.0], [0.0, 0.0]], [0, -1], 0.0, seed=1)
    assert not f & F_GATE


# ---------------------------------------------------------------- F3

def _bonus_seed():
    # A request whose two race exponentials are close, so the tuned logit stays small.
    for seed in range(1000):
        E = philox.race_exponentials(seed, 0, 0, 2)
        if abs(np.log(E[0] / E[1])) < 0.5:
            return seed, E
    raise AssertionError("no seed")


@pytest.mark.parametrize("window,fires", [(INSIDE, True), (OUTSIDE, False), ((0.0, 0.1 * BAND), True)])
def test_f3_bonus_race_band(window, fires):
    # A one-row request: its only row is the bonus row, a race over p with factor 1.
    seed, E = _bonus_seed()

    def gap(t):  # relative gap of the two keys p_x / E_x
        k = _softmax64(_f32([t, 0.0])) / E
        return abs(k[0] - k[1]) / k.max()

    t0 = float(np.log(E[0] / E[1]))  # keys equal here; the gap grows with t above it
    x, g = _tune(gap, t0, t0 + 0.5, window)
    f = _flags([[x, 0.0]], [[0.0, 0.0]], [-1], 0.0, seed)
    assert bool(f & F_RACE) == fires, (g, f)


def _residual_case(seed, t):
    """V = 3, tau = 0 (mu = q). Row 0 offers D = 0 with p(0)/q(0) = 1/3 and is rejected
    (the seed's u is above 1/2); the residual (p - q)+ is positive on tokens 1 and 2 only."""
    q = np.array([0.15, 0.40, 0.45])
    E = philox.race_exponentials(seed, 0, 0, 3)
    w1 = 0.10 / (1.0 + E[2] / E[1])  # tokens 1 and 2 tie when w2 / w1 = E2 / E1
    p = np.array([0.05, 0.40 + w1, 0.45 + (0.10 - w1)])
    tl = [[float(np.float32(np.log(p[0]))), float(np.float32(np.log(p[1]))), t], [4.0, -4.0, -4.0]]
    dl = [[float(x) for x in np.float32(np.log(q))], [0.0, 0.0, 0.0]]
    return tl, dl, E


def _residual_gap(seed, t):
    """(signed relative gap, factor c) of the residual race's two best keys. The gap is
    positive when token 2 leads, so it increases with token 2's logit t."""
    tl, dl, E = _residual_case(seed, t)
    p, q = _softmax64(_f32(tl[0])), _softmax64(_f32(dl[0]))
    w = np.maximum(p - q, 0.0)
    k = w / E
    assert w[0] == 0.0 and w[1] > 0.0 and w[2] > 0.0
    c = max(1.0, (p[1] + q[1]) / w[1], (p[2] + q[2]) / w[2])
    return (k[2] - k[1]) / max(k[1], k[2]), c


def _residual_seed():
    for seed in range(1000):
        if philox.accept_uniform(seed, 0, 0) > 0.5:
            E = philox.race_exponentials(seed, 0, 0, 3)
            if 0.8 < E[2] / E[1] < 1.25:
                return seed
    raise AssertionError("no seed")


@pytest.mark.parametrize("lo,hi,fires", [
    (0.5, 0.9, True),      # inside 1e-6 * c
    (1.1, 1.5, False),     # outside 1e-6 * c
    (None, None, True),    # between 1e-6 and 1e-6 * c: fires only through the factor
])
def test_f3_residual_race_band_with_factor(lo, hi, fires):
    seed = _residual_seed()
    _, _, E = _residual_case(seed, 0.0)
    t_tie = float(np.log(0.45 + (0.10 - 0.10 / (1.0 + E[2] / E[1]))))
    _, c = _residual_gap(seed, t_tie)
    assert c > 10.0  # the factor is large enough to separate the bands
    window = (2.0 * BAND, 0.5 * c * BAND) if lo is None else (lo * c * BAND, hi * c * BAND)
    x, g = _tune(lambda t: _residual_gap(seed, t)[0], t_tie - 1e-2, t_tie + 1e-2, window)
    gg, cc = _residual_gap(seed, x)
    assert abs(cc / c - 1.0) < 1e-3
    tl, dl, _ = _residual_case(seed, x)
    res = verify_request(_f32(tl), _f32(dl), np.array([0, -1]), 1.0, 0.0, seed, 0)
    assert res.rows[0].verdict == 2  # rejected: the residual race decides the token
    assert bool(res.flags & F_RACE) == fires, (gg, cc, res.flags)


# ---------------------------------------------------------------- F4

@pytest.mark.parametrize("window,sign,fires", [(INSIDE, 1, True), (INSIDE, -1, True),
                                              (OUTSIDE, 1, False), (OUTSIDE, -1, False)])
def test_f4_support_band(window, sign, fires):
    # V = 3, tau = 0.25: D = 0 has q = 0.1 (NULL, far from tau); token 2's q is tuned near tau.
    # p = (0.6, 0.2, 0.2) gives a residual on token 0 alone, far from empty, so only the
    # q_2 ~ tau condition can fire F4.
    tau = float(np.float32(0.25))
    tl = [[float(x) for x in np.float32(np.log([0.6, 0.2, 0.2]))], [4.0, -4.0, -4.0]]

    def dl_of(c):
        return [[float(np.float32(np.log(0.1))), float(np.float32(np.log(0.65))), c], [0.0, 0.0, 0.0]]

    def margin(c):  # sign * (q_2 - tau)
        return sign * (_softmax64(_f32(dl_of(c)[0]))[2] - tau)

    lo, hi = (np.log(0.2), np.log(0.3)) if sign > 0 else (-np.log(0.3), -np.log(0.2))
    x, m = _tune(lambda v: margin(sign * v), lo, hi, window)
    c = sign * x
    dl = dl_of(c)
    q = _softmax64(_f32(dl[0]))
    assert abs(q[0] - tau) > 0.1 and abs(q[1] - tau) > 0.1
    res = verify_request(_f32(tl), _f32(dl), np.array([0, -1]), 1.0, tau, 1, 0)
    assert res.rows[0].verdict == 3  # NULL: a residual race
    assert not res.flags & F_GATE
    assert bool(res.flags & F_SUPPORT) == fires, (m, res.flags)


@pytest.mark.parametrize("window,fires", [(INSIDE, True), (OUTSIDE, False)])
def test_f4_small_residual_mass(window, fires):
    # V = 3, tau = 0.1, D = 2 with q_2 = eps < tau (NULL) and p_2 = 0. Tokens 0 and 1 keep
    # q = (1 - eps)/2 each against p = 1/2, so the residual mass is exactly eps.
    tau = float(np.float32(0.1))
    tl = [[0.0, 0.0, -np.inf], [4.0, -4.0, -4.0]]

    def dl_of(c):
        return [[0.0, 0.0, c], [0.0, 0.0, 0.0]]

    def mass(c):
        p, q = _softmax64(_f32(tl[0])), _softmax64(_f32(dl_of(c)[0]))
        return float(np.maximum(p - np.where(q >= tau, q, 0.0), 0.0).sum())

    x, m = _tune(mass, -20.0, -10.0, window)
    res = verify_request(_f32(tl), _f32(dl_of(x)), np.array([2, -1]), 1.0, tau, 1, 0)
    assert res.rows[0].verdict == 3
    assert bool(res.flags & F_SUPPORT) == fires, (m, res.flags)


def test_greedy_requests_are_never_flagged():
    # Every quantity sits on its boundary, but T = 0 draws nothing.
    f = _flags([[0.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 0.0]], [0, -1], 0.5, seed=3, T=0.0)
    assert f == 0
