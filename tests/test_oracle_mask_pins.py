"""Pins for the sliding-window and packed variable-length oracle.

* Brute force on tiny inputs: each row's visible keys listed by hand from the
  definition (i - wl <= j <= i + wr, causal j <= i), softmax and weighted sum
  computed row by row with math.exp, independent of the oracle's vectorised mask.
* Reductions to the pinned dense oracle: unbounded windows and windows wider than
  the sequence give plain (causal) attention; one packed sequence is the dense case.
* Closed forms: window_left = 0 with causal means each row sees only itself
  (O_i = v_i, lse_i = s_ii); identical keys give the mean of the visible values and
  lse = s + ln(#visible) with #visible from the window.
* Packing: permuting whole sequences permutes their outputs.
* Planted mistakes (window edge off by one, window side swapped) must fail the brute force.
"""
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(777)


def brute(q, k, v, scale, causal, wl, wr):
    N, D = q.shape
    o = np.zeros((N, v.shape[1]))
    lse = np.full(N, -math.inf)
    for i in range(N):
        js = [j for j in range(k.shape[0])
              if (not causal or j <= i) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
        if not js:
            continue
        s = [scale * sum(q[i, d] * k[j, d] for d in range(D)) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = sum(e)
        for idx, j in enumerate(js):
            o[i] += e[idx] / den * v[j]
        lse[i] = m + math.log(den)
    return o, lse


CASES = [(False, -1, -1), (True, -1, -1), (True, 3, -1), (False, 2, 1), (False, 0, 4),
         (True, 0, 0), (False, -1, 2), (False, 5, -1), (True, 1, 7)]


@pytest.mark.parametrize("causal,wl,wr", CASES)
def test_brute_force(causal, wl, wr):
    N, D = 11, 3
    q, k, v = RNG.standard_normal((N, D)), RNG.standard_normal((N, D)), RNG.standard_normal((N, D))
    o, lse = oracle.attention_window(q[None, None], k[None, None], v[None, None], 0.6, causal, wl, wr,
                                     row_block=4)
    ob, lb = brute(q, k, v, 0.6, causal, wl, wr)
    np.testing.assert_allclose(o[0, 0], ob, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lb, atol=1e-13)


@pytest.mark.parametrize("mistake", ["off_by_one", "sides_swapped"])
def test_planted_mistakes_fail_brute_force(monkeypatch, mistake):
    import oracle.masks as om
    good = om.visible

    def bad(rows, cols, causal, wl, wr):
        if mistake == "off_by_one":
            return good(rows, cols, causal, wl + 1 if wl >= 0 else wl, wr)
        return good(rows, cols, causal, wr, wl)

    monkeypatch.setattr(om, "visible", bad)
    N, D = 11, 3
    q, k, v = RNG.standard_normal((N, D)), RNG.standard_normal((N, D)), RNG.standard_normal((N, D))
    o, _ = oracle.attention_window(q[None, None], k[None, None], v[None, None], 0.6, False, 2, 0)
    ob, _ = brute(q, k, v, 0.6, False, 2, 0)
    assert np.max(np.abs(o[0, 0] - ob)) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_unbounded_and_wide_windows_are_plain_attention(causal):
    q, k, v = (RNG.standard_normal((2, 2, 40, 8)) for _ in range(3))
    ref = oracle.attention(q, k, v, 0.3, causal)
    for wl, wr in ((-1, -1), (40, 40), (1000, -1)):
        o, lse = oracle.attention_window(q, k, v, 0.3, causal, wl, wr)
        np.testing.assert_allclose(o, ref[0], atol=1e-13)
        np.testing.assert_allclose(lse, ref[1], atol=1e-13)


def test_window_zero_causal_sees_itself():
    q, k, v = (RNG.standard_normal((1, 3, 25, 8)) for _ in range(3))
    o, lse = oracle.attention_window(q, k, v, 0.4, True, 0, -1)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, 0.4 * np.sum(q * k, axis=-1), atol=1e-13)


@pytest.mark.parametrize("causal,wl,wr", [(False, 3, 2), (True, 4, -1), (False, 0, 5)])
def test_identical_keys_mean_and_log_count(causal, wl, wr):
    N, D = 30, 8
    q, v = RNG.standard_normal((N, D)), RNG.standard_normal((N, D))
    k = np.broadcast_to(RNG.standard_normal(D), (N, D)).copy()
    o, lse = oracle.attention_window(q[None, None], k[None, None], v[None, None], 0.25, causal, wl, wr)
    for i in range(N):
        js = [j for j in range(N) if (not causal or j <= i) and (wl < 0 or j >= i - wl)
              and (wr < 0 or j <= i + wr)]
        np.testing.assert_allclose(o[0, 0, i], v[js].mean(0), atol=1e-13)
        assert abs(lse[0, 0, i] - (0.25 * q[i] @ k[0] + math.log(len(js)))) < 1e-12


def test_varlen_one_sequence_is_dense():
    q, k, v = (RNG.standard_normal((3, 50, 8)) for _ in range(3))
    o, lse = oracle.attention_varlen(q, k, v, [0, 50], 0.3, True, 7, -1)
    od, ld = oracle.attention_window(q[None], k[None], v[None], 0.3, True, 7, -1)
    np.testing.assert_allclose(o, od[0], atol=1e-14)
    np.testing.assert_allclose(lse, ld[0], atol=1e-14)


def test_varlen_sequences_are_independent_and_permutable():
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (RNG.standard_normal((2, cu[-1], 8)) for _ in range(3))
    o, lse = oracle.attention_varlen(q, k, v, cu, 0.5, True)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if b > a:
            od, ld = oracle.attention(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.5, True)
            np.testing.assert_allclose(o[:, a:b], od[0], atol=1e-14)
            np.testing.assert_allclose(lse[:, a:b], ld[0], atol=1e-14)
    order = [4, 2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order]).astype(int)
    cu2 = np.concatenate([[0], np.cumsum([lens[s] for s in order])])
    o2, l2 = oracle.attention_varlen(q[:, idx], k[:, idx], v[:, idx], cu2, 0.5, True)
    np.testing.assert_allclose(o2, o[:, idx], atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, idx], atol=1e-14)


def test_window_row_block_and_workers_do_not_matter():
    """The thread pool and the row blocking are plumbing: any split of the independent
    (b, h, row-block) units gives the same rows (up to the BLAS's own blocking)."""
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((2, 3, 75, 8)) for _ in range(3))
    for causal, wl, wr in ((True, 10, -1), (False, 7, 3), (False, -1, -1)):
        o1, l1 = oracle.attention_window(q, k, v, 0.4, causal, wl, wr, row_block=1024)
        o2, l2 = oracle.attention_window(q, k, v, 0.4, causal, wl, wr, row_block=7, workers=5)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
    cu = np.array([0, 20, 21, 75])
    o1, l1 = oracle.attention_varlen(q[0], k[0], v[0], cu, 0.4, True)
    o2, l2 = oracle.attention_varlen(q[0], k[0], v[0], cu, 0.4, True, workers=3)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
