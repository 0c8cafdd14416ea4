"""Plain fp64 CPU oracle for the two reductions the pages put beside attention: the
online-softmax normaliser (m, d) and Welford's running moments (n, mu, M2), each over
the rows of a matrix.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The library's device path never
calls it, and it imports nothing from the library: the two share no code.

Sources ("Learning FlashAttention the Hard Way -- Part 1", cloudrift.ai):

* the safe softmax and its normaliser: m = max_j x_j and d = sum_j e^{x_j - m}
  (section "Softmax Looks Like It Breaks the Rules"); the carrier (m, d), the
  injection (x, 1), the combine that rescales both sides to the larger maximum and
  the identity (-inf, 0) (section "Online Softmax Reparametrization");
* Welford's carrier (n, mu, M2): count, mean and sum of squared deviations from
  the mean; the injection (1, x, 0), the pairwise merge of Chan, Golub and LeVeque
  and the identity (0, 0, 0); the variance M2 / n (population) or M2 / (n - 1)
  (sample) read off the final triple (section "The Same Move: Welford's Variance").

`softmax_stats` and `moments` (and their prefix scans) are the definitions, evaluated
directly (max, then the sum of shifted exponentials; mean, then the sum of squared
deviations), a whole row (or prefix) at a time. The inject / combine functions are the monoid steps in the pages' notation, for
tests that fold them in arbitrary brackets and check the fold against the definitions.

The pages print the merges' formulas only as images; the readings taken are the
standard forms they describe in words: for (m, d), m = max(m_a, m_b) and
d = d_a e^{m_a - m} + d_b e^{m_b - m}, the identity (-inf, 0) contributing nothing;
for (n, mu, M2), n = n_a + n_b, mu = (n_a mu_a + n_b mu_b) / n and
M2 = M2_a + M2_b + (mu_a - mu_b)^2 n_a n_b / n, the identity (0, 0, 0) contributing
nothing.
"""
from __future__ import annotations

import math

import numpy as np

from .fp64 import NEG_INF, _f64


# --------------------------------------------------------------------------- definitions
def softmax_stats(x):
    """Per row of x [rows, n]: m = max_j x_j and d = sum_j e^{x_j - m}, in float64.

    A row with no element, or whose elements are all -inf, is the identity (-inf, 0).
    Returns (m [rows], d [rows])."""
    x = _f64(x)
    rows = x.shape[0]
    m = np.full(rows, NEG_INF)
    d = np.zeros(rows)
    if x.ndim != 2 or x.shape[1] == 0:
        return m, d
    m = x.max(axis=1)                          # pass 1: the maximum
    live = m > NEG_INF
    e = np.exp(x[live] - m[live, None])        # pass 2: shifted exponentials ...
    d[live] = e.sum(axis=1)                    # ... and their sum
    return m, d


def log_sum_exp(x):
    """ln sum_j e^{x_j} per row, read from the normaliser as m + ln d (-inf if empty)."""
    m, d = softmax_stats(x)
    out = np.full(m.shape, NEG_INF)
    live = d > 0
    out[live] = m[live] + np.log(d[live])
    return out


def moments(x):
    """Per row of x [rows, n]: count n, mean mu = (1/n) sum_j x_j and
    M2 = sum_j (x_j - mu)^2 (the stable two-pass form), in float64.

    A row with no element is the identity (0, 0, 0). Returns (count, mu, M2), each [rows]."""
    x = _f64(x)
    rows = x.shape[0]
    n = x.shape[1] if x.ndim == 2 else 0
    count = np.full(rows, float(n))
    if n == 0:
        return count, np.zeros(rows), np.zeros(rows)
    mu = x.sum(axis=1) / n                     # pass 1: the mean
    m2 = ((x - mu[:, None]) ** 2).sum(axis=1)  # pass 2: squared deviations from it
    return count, mu, m2


def variance(x, ddof: int = 0):
    """M2 / (n - ddof) per row: population variance (ddof 0) or sample variance (1)."""
    count, _, m2 = moments(x)
    return m2 / (count - ddof)


# --------------------------------------------------------------------------- prefix scans
# A prefix sum is one more re-bracketing that any monoid allows (section "Wrap-Up",
# first point): the inclusive scan of a row is, at every position j, the reduction of
# elements 0..j. These are that definition, each prefix reduced from scratch (O(n^2)
# per row, for test sizes).
def softmax_stats_scan(x):
    """Per row of x [rows, n] and position j: m[r, j] = max_{i<=j} x[r, i] and
    d[r, j] = sum_{i<=j} e^{x[r, i] - m[r, j]}; a prefix of only -inf is (-inf, 0).
    Returns (m, d), each [rows, n] float64."""
    x = _f64(x)
    rows, n = x.shape
    m = np.full((rows, n), NEG_INF)
    d = np.zeros((rows, n))
    for j in range(n):
        mj, dj = softmax_stats(x[:, :j + 1])
        m[:, j], d[:, j] = mj, dj
    return m, d


def moments_scan(x):
    """Per row of x [rows, n] and position j: the mean and M2 of x[r, 0..j] (count
    j + 1). Returns (mean, m2), each [rows, n] float64."""
    x = _f64(x)
    rows, n = x.shape
    mean = np.zeros((rows, n))
    m2 = np.zeros((rows, n))
    for j in range(n):
        _, mu, q = moments(x[:, :j + 1])
        mean[:, j], m2[:, j] = mu, q
    return mean, m2


# --------------------------------------------------------------------------- monoid steps
def softmax_identity():
    return (NEG_INF, 0.0)


def softmax_inject(x: float):
    """One score enters as (x, 1): e^{x - x} = 1."""
    return (float(x), 1.0)


def softmax_combine(a, b):
    """(m_a, d_a) + (m_b, d_b): both denominators rescaled to the larger maximum."""
    (ma, da), (mb, db) = a, b
    m = max(ma, mb)
    if m == NEG_INF:
        return softmax_identity()
    return (m, da * math.exp(ma - m) + db * math.exp(mb - m))


def welford_identity():
    return (0.0, 0.0, 0.0)


def welford_inject(x: float):
    """One sample enters as (1, x, 0)."""
    return (1.0, float(x), 0.0)


def welford_combine(a, b):
    """Chan-Golub-LeVeque merge of two disjoint partials."""
    (na, mua, m2a), (nb, mub, m2b) = a, b
    n = na + nb
    if n == 0:
        return welford_identity()
    delta = mub - mua
    mu = (na * mua + nb * mub) / n
    return (n, mu, m2a + m2b + delta * delta * na * nb / n)
