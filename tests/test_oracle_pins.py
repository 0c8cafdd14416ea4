"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Every check here is independent of the oracle's own formula: hand-derived
closed forms (tests/golden), closed forms that hold for whole families of
inputs, an independent library routine for the textbook special case, the
algebraic laws of the (m, d, o) combine, and brute force over every bracketing
and order on tiny inputs. The last group plants plausible mistakes in copies
of the oracle and checks that some pin catches each of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle import fp64 as oa
from tests.conftest import exact, exact_array, load_golden

TIGHT = 1e-12


def _golden_inputs(g):
    q = exact_array(g["q"])[None, None]
    k = exact_array(g["k"])[None, None]
    v = exact_array(g["v"])[None, None]
    return q, k, v, exact(g["scale"])


# ---------------------------------------------------------------- hand-derived golden cases
@pytest.mark.parametrize("causal", [False, True])
def test_golden_two_rows(causal):
    g = load_golden("two_rows_scaled.json")
    q, k, v, scale = _golden_inputs(g)
    exp = g["expected"]["causal" if causal else "noncausal"]
    o, lse = oracle.attention(q, k, v, scale, causal=causal)
    np.testing.assert_allclose(o[0, 0], exact_array(exp["o"]), rtol=0, atol=TIGHT)
    np.testing.assert_allclose(lse[0, 0], exact_array(exp["lse"]), rtol=0, atol=TIGHT)


def test_golden_huge_scores_need_max_subtraction():
    g = load_golden("huge_scores.json")
    q, k, v, scale = _golden_inputs(g)
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.exp(1000.0))  # the naive form cannot even be evaluated
    o, lse = oracle.attention(q, k, v, scale)
    exp = g["expected"]["noncausal"]
    np.testing.assert_allclose(o[0, 0], exact_array(exp["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], exact_array(exp["lse"]), rtol=1e-15, atol=0)


@pytest.mark.parametrize("splits", [2, 4])
def test_golden_decode_partials(splits):
    g = load_golden("decode_partials_five_keys.json")
    q, k, v, scale = _golden_inputs(g)
    m, d, o = oracle.decode_partials(q, k, v, scale, splits)
    exp = g["expected"][f"splits_{splits}"]
    np.testing.assert_allclose(m[0], exact_array(exp["m"]), rtol=0, atol=TIGHT)
    np.testing.assert_allclose(d[0], exact_array(exp["d"]), rtol=0, atol=TIGHT)
    np.testing.assert_allclose(o[0], exact_array(exp["o"]), rtol=0, atol=TIGHT)
    om, lm = oracle.combine_partials(m, d, o)
    np.testing.assert_allclose(om, exact_array(g["expected"]["merged"]["o"]), rtol=0, atol=TIGHT)
    np.testing.assert_allclose(lm, exact_array(g["expected"]["merged"]["lse"]), rtol=0, atol=TIGHT)


# ---------------------------------------------------------------- textbook special case
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,D", [(1, 8), (7, 16), (33, 64), (130, 128)])
def test_matches_torch_sdpa_fp64(causal, N, D):
    g = torch.Generator().manual_seed(N * 1000 + D)
    q, k, v = (torch.randn(2, 3, N, D, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale, causal=causal, row_block=16)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    S = scale * (q @ k.transpose(-1, -2))
    if causal:
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_that_value(causal):
    """All v_j equal v: every row's weights sum to one, so every output row is v."""
    rng = np.random.default_rng(11)
    N, D = 50, 16
    q = rng.standard_normal((1, 2, N, D)) * 4
    k = rng.standard_normal((1, 2, N, D)) * 4
    vrow = rng.standard_normal(D)
    v = np.broadcast_to(vrow, (1, 2, N, D)).copy()
    o, _ = oracle.attention(q, k, v, 0.3, causal=causal)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    """All k_j equal: every visible score is the same s_i, weights are uniform,
    o_i is the mean of the visible v_j and lse_i = s_i + ln(#visible)."""
    rng = np.random.default_rng(12)
    N, D = 40, 8
    q = rng.standard_normal((1, 1, N, D))
    krow = rng.standard_normal(D)
    k = np.broadcast_to(krow, (1, 1, N, D)).copy()
    v = rng.standard_normal((1, 1, N, D))
    scale = 0.7
    o, lse = oracle.attention(q, k, v, scale, causal=causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n_vis].mean(axis=0), rtol=0, atol=1e-12)
        s_i = scale * float(q[0, 0, i] @ krow)
        assert abs(lse[0, 0, i] - (s_i + math.log(n_vis))) < 1e-12


def test_single_key():
    """One visible key: the output is that key's value and lse is its score."""
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, 1, 1, 4)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, 1.3)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 1.3 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14
    q, k, v = (rng.standard_normal((1, 1, 9, 4)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, 1.3, causal=True)  # causal row 0 sees key 0 only
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 1.3 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14


def test_row_shift_invariance():
    """Adding a per-row constant to every score leaves O unchanged and shifts lse
    by that constant (multiply top and bottom by e^{-c}). Built by appending a
    column: Q[i, D] = c_i, K[j, D] = kappa, so s_ij gains scale * c_i * kappa."""
    rng = np.random.default_rng(14)
    N, D = 30, 8
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    c = rng.standard_normal(N) * 20
    kappa, scale = 3.0, 0.5
    q2 = np.concatenate([q, c[None, None, :, None]], axis=-1)
    k2 = np.concatenate([k, np.full((1, 1, N, 1), kappa)], axis=-1)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, scale, causal=causal)
        o2, l2 = oracle.attention(q2, k2, v, scale, causal=causal)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-11)
        np.testing.assert_allclose(l2[0, 0], l1[0, 0] + scale * kappa * c, rtol=0, atol=1e-10)


def test_key_permutation_invariance():
    """Permuting the key/value pairs together changes nothing (the combine commutes)."""
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((2, 2, 25, 16)) for _ in range(3))
    perm = rng.permutation(25)
    o1, l1 = oracle.attention(q, k, v, 0.25)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_base2_twist_is_the_same_function():
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((1, 2, 20, 8)) * 3 for _ in range(3))
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, 0.4, causal=causal)
        o2, l2 = oracle.attention_base2(q, k, v, 0.4, causal=causal)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_row_block_and_workers_do_not_matter():
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((2, 2, 70, 8)) for _ in range(3))
    o1, l1 = oracle.attention(q, k, v, 0.5, causal=True, row_block=1024)
    o2, l2 = oracle.attention(q, k, v, 0.5, causal=True, row_block=9, workers=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    rows = [(1, 0, 0), (0, 1, 69), (1, 1, 33)]
    o3, l3 = oracle.attention_selected_rows(q, k, v, 0.5, True, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o3[n], o1[b, h, i], rtol=0, atol=1e-13)
        assert abs(l3[n] - l1[b, h, i]) < 1e-13


def test_fully_masked_row_is_identity():
    P, m, d = oracle.safe_softmax_rows(np.full((2, 5), -np.inf))
    assert np.all(P == 0) and np.all(np.isneginf(m)) and np.all(d == 0)
    assert np.all(np.isneginf(oracle.logsumexp_from_state(m, d)))


# ---------------------------------------------------------------- the (m, d, o) monoid
def _random_tree(n, draw_bits):
    """A random full binary bracketing of leaves 0..n-1, as nested tuples."""
    if n == 1:
        return 0
    split = 1 + draw_bits(n - 1)
    left = _random_tree(split, draw_bits)
    right = _random_tree(n - split, draw_bits)
    return (left, _shift(right, split))


def _shift(t, by):
    return t + by if isinstance(t, int) else (_shift(t[0], by), _shift(t[1], by))


def _fold_tree(t, states):
    if isinstance(t, int):
        return states[t]
    return oracle.combine(_fold_tree(t[0], states), _fold_tree(t[1], states))


def _all_trees(lo, hi):
    if hi - lo == 1:
        yield lo
        return
    for mid in range(lo + 1, hi):
        for a in _all_trees(lo, mid):
            for b in _all_trees(mid, hi):
                yield (a, b)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.integers(0, 2**31 - 1), st.data())
def test_random_bracketings_equal_the_plain_formula(n, seed, data):
    """Folding the injected single-key states (s_j, 1, v_j) under any bracketing
    reads out the same row as the materialised softmax (associativity)."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n) * 10
    V = rng.standard_normal((n, 5))
    tree = _random_tree(n, lambda k: data.draw(st.integers(0, k - 1)))
    u = _fold_tree(tree, [oracle.inject(s[j], V[j]) for j in range(n)])
    o, lse = oracle.readout(u)
    P, m, d = oracle.safe_softmax_rows(s[None])
    np.testing.assert_allclose(o, (P @ V)[0], rtol=1e-12, atol=1e-12)
    assert abs(lse - oracle.logsumexp_from_state(m, d)[0]) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_brute_force_every_order_and_bracketing(n):
    rng = np.random.default_rng(100 + n)
    s = rng.standard_normal(n) * 5
    V = rng.standard_normal((n, 3))
    P, m, d = oracle.safe_softmax_rows(s[None])
    want_o, want_l = (P @ V)[0], oracle.logsumexp_from_state(m, d)[0]
    trees = list(_all_trees(0, n))
    assert len(trees) == math.comb(2 * (n - 1), n - 1) // n  # Catalan number C_{n-1}
    for perm in itertools.permutations(range(n)):
        states = [oracle.inject(s[j], V[j]) for j in perm]
        for t in trees:
            o, lse = oracle.readout(_fold_tree(t, states))
            np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-13)
            assert abs(lse - want_l) < 1e-13


def test_identity_laws_and_block_state():
    rng = np.random.default_rng(21)
    e = oracle.identity_state(4)
    s = rng.standard_normal(7) * 3
    V = rng.standard_normal((7, 4))
    u = oracle.block_state(s, V)
    for w in (oracle.combine(u, e), oracle.combine(e, u)):
        assert w[0] == u[0] and w[1] == u[1]
        np.testing.assert_array_equal(w[2], u[2])
    ee = oracle.combine(e, e)
    assert ee[0] == -math.inf and ee[1] == 0.0 and not np.any(ee[2])
    # padding with masked keys (-inf scores) changes nothing
    u_pad = oracle.block_state(np.concatenate([s, [-np.inf] * 3]), np.concatenate([V, rng.standard_normal((3, 4))]))
    assert u_pad[0] == u[0] and abs(u_pad[1] - u[1]) < 1e-15
    np.testing.assert_allclose(u_pad[2], u[2], atol=1e-15)
    # range: the argmax term is e^0 = 1, so 1 <= d <= n
    assert 1.0 <= u[1] <= 7.0
    # commutativity
    u2 = oracle.block_state(rng.standard_normal(5), rng.standard_normal((5, 4)))
    a, b = oracle.combine(u, u2), oracle.combine(u2, u)
    assert a[0] == b[0] and abs(a[1] - b[1]) < 1e-14
    np.testing.assert_allclose(a[2], b[2], atol=1e-14)
    # a block's state equals the fold of its single-key injections
    f = e
    for j in range(7):
        f = oracle.combine(f, oracle.inject(s[j], V[j]))
    assert f[0] == u[0] and abs(f[1] - u[1]) < 1e-13
    np.testing.assert_allclose(f[2], u[2], atol=1e-13)


@pytest.mark.parametrize("L,splits", [(1, 1), (100, 1), (100, 7), (100, 64), (5, 8), (512, 64)])
def test_decode_partials_merge_to_attention(L, splits):
    rng = np.random.default_rng(L * 10 + splits)
    q = rng.standard_normal((2, 3, 1, 16))
    k = rng.standard_normal((2, 3, L, 16)) * 2
    v = rng.standard_normal((2, 3, L, 16))
    m, d, o = oracle.decode_partials(q, k, v, 0.25, splits)
    valid = ~np.isneginf(m)
    assert np.all(d[valid] >= 1.0) and np.all(d[~valid] == 0.0)
    c = -(-L // splits)
    for s, (j0, j1) in enumerate(oracle.split_bounds(L, splits)):
        assert np.all(d[:, s] <= max(j1 - j0, 0) + 1e-12) and j1 - j0 <= c
    om, lm = oracle.combine_partials(m, d, o)
    oref, lref = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(om, oref.reshape(6, 16), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lref.reshape(6), rtol=0, atol=1e-12)
    # any order of the partials merges to the same result
    perm = rng.permutation(splits)
    om2, lm2 = oracle.combine_partials(m[:, perm], d[:, perm], o[:, perm])
    np.testing.assert_allclose(om2, om, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm2, lm, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes must be caught
def _pins_pass() -> bool:
    """Run the golden and closed-form pins against the (possibly mutated) oracle."""
    try:
        for causal in (False, True):
            test_golden_two_rows(causal)
            test_identical_keys_give_mean_of_visible_values(causal)
        test_golden_huge_scores_need_max_subtraction()
        test_golden_decode_partials(2)
        test_golden_decode_partials(4)
        test_matches_torch_sdpa_fp64(True, 7, 16)
        return True
    except (AssertionError, FloatingPointError, ValueError):
        return False


def _mut_rows_transposed(qh, kh, vh, scale, causal, r0, r1):
    S = scale * (kh @ qh.T)[r0:r1]  # scores transposed
    if causal:
        S = np.where(np.arange(kh.shape[0])[None] <= np.arange(r0, r1)[:, None], S, -np.inf)
    P, m, d = oa.safe_softmax_rows(S)
    return P @ vh, oa.logsumexp_from_state(m, d)


def _mut_rows_no_scale(qh, kh, vh, scale, causal, r0, r1):
    return _ORIG_ROWS(qh, kh, vh, 1.0, causal, r0, r1)


def _mut_rows_reversed_mask(qh, kh, vh, scale, causal, r0, r1):
    S = scale * (qh[r0:r1] @ kh.T)
    if causal:
        S = np.where(np.arange(kh.shape[0])[None] >= np.arange(r0, r1)[:, None], S, -np.inf)
    P, m, d = oa.safe_softmax_rows(S)
    return P @ vh, oa.logsumexp_from_state(m, d)


def _mut_softmax_no_max(S):
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(np.asarray(S, dtype=np.float64))
        d = E.sum(axis=-1)
        return E / d[..., None], np.zeros(d.shape), d


def _mut_lse_log2(m, d):
    with np.errstate(divide="ignore"):
        return np.where(np.asarray(d) > 0, np.asarray(m) + np.log2(d), -np.inf)


def _mut_combine_wrong_sign(ua, ub):
    ma, da, oa_ = ua
    mb, db, ob = ub
    if ma >= mb:
        if mb == -math.inf:
            return ua
        f = math.exp(ma - mb)  # sign flipped
        return (ma, da + db * f, oa_ + ob * f)
    f = math.exp(mb - ma)
    return (mb, db + da * f, ob + oa_ * f)


def _mut_combine_drops_o_rescale(ua, ub):
    ma, da, oa_ = ua
    mb, db, ob = ub
    if ma >= mb:
        if mb == -math.inf:
            return ua
        f = math.exp(mb - ma)
        return (ma, da + db * f, oa_ + ob)
    f = math.exp(ma - mb)
    return (mb, db + da * f, ob + oa_)


_ORIG_ROWS = oa._attention_rows


@pytest.mark.parametrize("target,mutant", [
    ("_attention_rows", _mut_rows_transposed),
    ("_attention_rows", _mut_rows_no_scale),
    ("_attention_rows", _mut_rows_reversed_mask),
    ("safe_softmax_rows", _mut_softmax_no_max),
    ("logsumexp_from_state", _mut_lse_log2),
    ("combine", _mut_combine_wrong_sign),
    ("combine", _mut_combine_drops_o_rescale),
])
def test_pins_catch_planted_mistakes(monkeypatch, target, mutant):
    assert _pins_pass(), "the unmutated oracle must pass its pins"
    monkeypatch.setattr(oa, target, mutant)
    monkeypatch.setattr(oracle, target, mutant, raising=False)
    assert not _pins_pass(), f"planting {mutant.__name__} went unnoticed"
