"""Pins for the reduction oracle (online-softmax normaliser and Welford moments).

None of these reuses the oracle's formulas:
* exact rational arithmetic (fractions + the standard library's statistics module)
  for the mean and the sum of squared deviations on dyadic data;
* brute force with Python's math.exp and math.fsum, and SciPy's logsumexp (an
  independent library) for the normaliser;
* closed forms: constant rows, 1..n, two values, a large common offset that defeats
  the naive one-pass variance, scores that overflow without the maximum shift,
  -inf entries (the identity) and empty rows;
* the pages' monoid claim: folding the injections with the combine in random
  bracketings and orders gives the definition;
* prefix scans: the last position equals the (pinned) reduction, closed forms per
  prefix (1..j, constant and geometric rows, -inf prefixes), exact rational moments of
  every prefix, and a Blelloch up-sweep / down-sweep scan built from the monoid steps;
* planted mistakes, each of which must fail at least one pin.
"""
import math
import random
import statistics
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle.monoids as om

RNG = np.random.default_rng(2024)


# ------------------------------------------------------------------ pins as functions
def pin_softmax_brute(stats):
    x = RNG.standard_normal((6, 13)) * 4
    m, d = stats(x)
    for r in range(x.shape[0]):
        mr = max(x[r])
        assert m[r] == mr
        assert abs(d[r] - math.fsum(math.exp(v - mr) for v in x[r])) <= 1e-13 * d[r]


def pin_softmax_scipy(stats):
    x = RNG.standard_normal((5, 1000)) * 20
    m, d = stats(x)
    np.testing.assert_allclose(m + np.log(d), logsumexp(x, axis=1), rtol=0, atol=1e-12)


def pin_softmax_closed_forms(stats):
    m, d = stats(np.full((2, 7), 3.25))
    assert np.all(m == 3.25) and np.all(d == 7.0)          # constant row: d = n
    m, d = stats(np.array([[1000.0, 1001.0]]))              # e^1001 overflows unshifted
    assert m[0] == 1001.0 and abs(d[0] - (1 + math.exp(-1))) <= 1e-15
    m, d = stats(np.array([[2.0, math.log(2.0) + 2.0, -math.inf]]))
    assert m[0] == 2.0 + math.log(2.0) and abs(d[0] - 1.5) <= 1e-15   # -inf adds nothing
    m, d = stats(np.array([[-math.inf, -math.inf]]))
    assert m[0] == -math.inf and d[0] == 0.0                # all masked: the identity
    m, d = stats(np.zeros((3, 0)))
    assert np.all(m == -math.inf) and np.all(d == 0.0)      # empty rows: the identity


def _exact_moments(vals):
    fr = [Fraction(v) for v in vals]
    mu = statistics.mean(fr)
    return mu, statistics.pvariance(fr) * len(fr)


def pin_moments_exact(moments):
    # dyadic data: every value, the exact mean and the exact M2 are checked exactly
    # against rational arithmetic (within fp64 rounding of the results)
    x = np.round(RNG.standard_normal((5, 33)) * 64) / 8
    n, mu, m2 = moments(x)
    assert np.all(n == 33)
    for r in range(x.shape[0]):
        emu, em2 = _exact_moments(x[r])
        assert abs(mu[r] - float(emu)) <= 1e-15 * max(1.0, abs(float(emu)))
        assert abs(m2[r] - float(em2)) <= 1e-13 * float(em2)


def pin_moments_closed_forms(moments):
    k = 100
    n, mu, m2 = moments(np.arange(1, k + 1, dtype=float)[None])
    assert mu[0] == (k + 1) / 2 and m2[0] == k * (k * k - 1) / 12   # 1..n
    n, mu, m2 = moments(np.full((1, 9), -7.5))
    assert mu[0] == -7.5 and m2[0] == 0.0                           # constant row
    n, mu, m2 = moments(np.array([[3.0, 11.0]]))
    assert mu[0] == 7.0 and m2[0] == 32.0                           # (a - b)^2 / 2
    # a common offset of 1e9: the naive sum-of-squares formula loses every digit here
    n, mu, m2 = moments(np.array([[1e9, 1e9 + 1, 1e9 + 2, 1e9 + 3]]))
    assert mu[0] == 1e9 + 1.5 and m2[0] == 5.0
    n, mu, m2 = moments(np.zeros((2, 0)))
    assert np.all(n == 0) and np.all(mu == 0) and np.all(m2 == 0)   # empty: the identity


def pin_variance_bessel(variance):
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    assert variance(x)[0] == 1.25 and abs(variance(x, ddof=1)[0] - 5.0 / 3.0) <= 1e-15


def _random_fold(items, inject, combine, identity, rnd):
    """Fold the injections of `items`, shuffled, in a random bracketing, with identities
    sprinkled in."""
    states = [inject(v) for v in items] + [identity() for _ in range(rnd.randint(0, 3))]
    rnd.shuffle(states)
    while len(states) > 1:
        i = rnd.randrange(len(states) - 1)
        states[i:i + 2] = [combine(states[i], states[i + 1])]
    return states[0] if states else identity()


def pin_softmax_fold(stats, combine=om.softmax_combine):
    rnd = random.Random(5)
    for _ in range(30):
        x = RNG.standard_normal(rnd.randint(1, 40)) * 10
        m, d = _random_fold(list(x), om.softmax_inject, combine, om.softmax_identity, rnd)
        mr, dr = stats(x[None])
        assert m == mr[0] and abs(d - dr[0]) <= 1e-12 * dr[0]


def pin_welford_fold(moments, combine=om.welford_combine):
    rnd = random.Random(6)
    for _ in range(30):
        x = RNG.standard_normal(rnd.randint(1, 40)) * 3 + 5
        n, mu, m2 = _random_fold(list(x), om.welford_inject, combine, om.welford_identity, rnd)
        nr, mur, m2r = moments(x[None])
        assert n == nr[0] and abs(mu - mur[0]) <= 1e-13 * abs(mur[0])
        assert abs(m2 - m2r[0]) <= 1e-11 * m2r[0]


SOFTMAX_PINS = [pin_softmax_brute, pin_softmax_scipy, pin_softmax_closed_forms, pin_softmax_fold]
MOMENT_PINS = [pin_moments_exact, pin_moments_closed_forms, pin_welford_fold]


# ------------------------------------------------------------------ the oracle passes
@pytest.mark.parametrize("pin", SOFTMAX_PINS, ids=lambda p: p.__name__)
def test_softmax_stats_pins(pin):
    pin(om.softmax_stats)


@pytest.mark.parametrize("pin", MOMENT_PINS, ids=lambda p: p.__name__)
def test_moments_pins(pin):
    pin(om.moments)


def test_variance_bessel():
    pin_variance_bessel(om.variance)


def test_log_sum_exp_matches_scipy():
    x = RNG.standard_normal((4, 300)) * 30
    x[1, :] = -math.inf
    ref = logsumexp(x, axis=1)
    got = om.log_sum_exp(x)
    assert got[1] == -math.inf
    keep = [0, 2, 3]
    np.testing.assert_allclose(got[keep], ref[keep], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ planted mistakes
def _unshifted_stats(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        d = np.exp(x).sum(axis=1)
    return np.zeros(x.shape[0]), d  # "m = 0": no maximum shift


def _mean_shift_stats(x):  # shifts by the mean instead of the maximum
    x = np.asarray(x, dtype=np.float64)
    m = x.mean(axis=1)
    return m, np.exp(x - m[:, None]).sum(axis=1)


def _naive_moments(x):  # the one-pass sum-of-squares formula
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1]
    mu = x.sum(axis=1) / n
    return np.full(x.shape[0], float(n)), mu, (x * x).sum(axis=1) - n * mu * mu


def _biased_moments(x):  # deviations around the median instead of the mean
    x = np.asarray(x, dtype=np.float64)
    med = np.median(x, axis=1)
    return (np.full(x.shape[0], float(x.shape[1])), x.mean(axis=1),
            ((x - med[:, None]) ** 2).sum(axis=1))


def _fails_some(pins, impl, **kw):
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(impl, **kw) if kw else pin(impl)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            return True
    return False


@pytest.mark.parametrize("impl", [_unshifted_stats, _mean_shift_stats])
def test_planted_softmax_mistakes_fail(impl):
    assert _fails_some(SOFTMAX_PINS, impl)


@pytest.mark.parametrize("impl", [_naive_moments, _biased_moments])
def test_planted_moment_mistakes_fail(impl):
    assert _fails_some(MOMENT_PINS, impl)


def _combine_sign_flipped(a, b):
    (ma, da), (mb, db) = a, b
    m = max(ma, mb)
    if m == -math.inf:
        return (m, 0.0)
    return (m, da * math.exp(m - ma) + db * math.exp(m - mb))


def _combine_no_rescale(a, b):
    return (max(a[0], b[0]), a[1] + b[1])


def _welford_no_cross_term(a, b):
    (na, mua, m2a), (nb, mub, m2b) = a, b
    n = na + nb
    return (n, (na * mua + nb * mub) / n if n else 0.0, m2a + m2b)


def _welford_unweighted_mean(a, b):
    (na, mua, m2a), (nb, mub, m2b) = a, b
    n = na + nb
    if n == 0:
        return (0.0, 0.0, 0.0)
    if na == 0 or nb == 0:
        return a if nb == 0 else b
    d = mub - mua
    return (n, (mua + mub) / 2, m2a + m2b + d * d * na * nb / n)


@pytest.mark.parametrize("combine", [_combine_sign_flipped, _combine_no_rescale])
def test_planted_softmax_combine_mistakes_fail(combine):
    with pytest.raises((AssertionError, OverflowError)):
        pin_softmax_fold(om.softmax_stats, combine=combine)


@pytest.mark.parametrize("combine", [_welford_no_cross_term, _welford_unweighted_mean])
def test_planted_welford_combine_mistakes_fail(combine):
    with pytest.raises(AssertionError):
        pin_welford_fold(om.moments, combine=combine)


# ------------------------------------------------------------------ prefix scans
def pin_scan_last_is_reduction(scan_sm, scan_mo):
    x = RNG.standard_normal((4, 57)) * 7
    m, d = scan_sm(x)
    mr, dr = om.softmax_stats(x)
    assert np.array_equal(m[:, -1], mr) and np.allclose(d[:, -1], dr, rtol=1e-13)
    mean, m2 = scan_mo(x)
    _, mu, q = om.moments(x)
    assert np.allclose(mean[:, -1], mu, rtol=1e-14) and np.allclose(m2[:, -1], q, rtol=1e-12)


def pin_scan_closed_forms(scan_sm, scan_mo):
    k = 60
    j = np.arange(k)
    mean, m2 = scan_mo(np.arange(1, k + 1, dtype=float)[None])
    assert np.array_equal(mean[0], (j + 2) / 2)               # mean of 1..j+1
    assert np.allclose(m2[0], (j + 1) * ((j + 1) ** 2 - 1) / 12, rtol=1e-13, atol=0)
    m, d = scan_sm(np.full((1, k), -2.0))
    assert np.all(m == -2.0) and np.array_equal(d[0], j + 1.0)  # constant: d counts
    m, d = scan_sm((j * math.log(2.0))[None])                   # x_j = j ln 2, rising
    assert np.allclose(m[0], j * math.log(2.0), rtol=1e-15)
    assert np.allclose(d[0], 2.0 - 2.0 ** (-j), rtol=1e-13)   # sum_i 2^{i-j}
    m, d = scan_sm(np.array([[-math.inf, -math.inf, 1.0, -math.inf]]))
    assert list(m[0]) == [-math.inf, -math.inf, 1.0, 1.0] and list(d[0]) == [0.0, 0.0, 1.0, 1.0]


def pin_scan_exact_moments(scan_mo):
    x = np.round(RNG.standard_normal((2, 20)) * 16) / 4
    mean, m2 = scan_mo(x)
    for r in range(2):
        for j in range(20):
            emu, em2 = _exact_moments(x[r, :j + 1])
            assert abs(mean[r, j] - float(emu)) <= 1e-15 * max(1.0, abs(float(emu)))
            assert abs(m2[r, j] - float(em2)) <= 1e-13 * max(1.0, float(em2))


def _blelloch(items, inject, combine, identity):
    """Exclusive scan by the up-sweep / down-sweep of a balanced tree (Blelloch), then
    one more combine per element: a bracketing unlike the left fold of the definition."""
    n = 1
    while n < len(items):
        n *= 2
    a = [inject(v) for v in items] + [identity()] * (n - len(items))
    tree = list(a)
    step = 1
    while step < n:  # up-sweep
        for i in range(2 * step - 1, n, 2 * step):
            tree[i] = combine(tree[i - step], tree[i])
        step *= 2
    tree[n - 1] = identity()
    step = n // 2
    while step >= 1:  # down-sweep
        for i in range(2 * step - 1, n, 2 * step):
            left = tree[i - step]
            tree[i - step] = tree[i]
            tree[i] = combine(tree[i], left)
        step //= 2
    return [combine(tree[i], a[i]) for i in range(len(items))]


def pin_scan_blelloch(scan_sm, scan_mo):
    x = RNG.standard_normal(45) * 9
    m, d = scan_sm(x[None])
    st = _blelloch(list(x), om.softmax_inject, om.softmax_combine, om.softmax_identity)
    assert [s[0] for s in st] == list(m[0])
    assert np.allclose([s[1] for s in st], d[0], rtol=1e-12)
    mean, m2 = scan_mo(x[None] + 3)
    st = _blelloch(list(x + 3), om.welford_inject, om.welford_combine, om.welford_identity)
    assert np.allclose([s[1] for s in st], mean[0], rtol=1e-13)
    assert np.allclose([s[2] for s in st], m2[0], rtol=1e-11, atol=1e-12)


def test_scan_pins():
    pin_scan_last_is_reduction(om.softmax_stats_scan, om.moments_scan)
    pin_scan_closed_forms(om.softmax_stats_scan, om.moments_scan)
    pin_scan_exact_moments(om.moments_scan)
    pin_scan_blelloch(om.softmax_stats_scan, om.moments_scan)


def _exclusive_softmax_scan(x):  # planted: position j reduces 0..j-1
    m, d = om.softmax_stats_scan(x)
    x = np.asarray(x, dtype=float)
    m2 = np.concatenate([np.full((x.shape[0], 1), -math.inf), m[:, :-1]], axis=1)
    d2 = np.concatenate([np.zeros((x.shape[0], 1)), d[:, :-1]], axis=1)
    return m2, d2


def _running_max_only(x):  # planted: d not rescaled when the maximum moves
    x = np.asarray(x, dtype=float)
    m = np.maximum.accumulate(x, axis=1)
    d = np.cumsum(np.exp(x - m), axis=1)
    return m, d


@pytest.mark.parametrize("impl", [_exclusive_softmax_scan, _running_max_only])
def test_planted_scan_mistakes_fail(impl):
    failed = False
    for pin in (lambda: pin_scan_last_is_reduction(impl, om.moments_scan),
                lambda: pin_scan_closed_forms(impl, om.moments_scan),
                lambda: pin_scan_blelloch(impl, om.moments_scan)):
        try:
            pin()
        except AssertionError:
            failed = True
    assert failed
