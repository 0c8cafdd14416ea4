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
