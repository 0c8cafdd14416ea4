"""Pins for the fp64 backward oracle, independent of its own formulas.

The gradients are checked against what the forward definition fixes:
* central finite differences of L = sum(O * dO), with O from the forward oracle
  (pinned on its own), in random directions, on tiny shapes;
* invariants: the scores of a row may all shift by one constant without changing
  O, so sum_j dK_j = 0; the result is linear in dO; permuting keys and values
  together permutes dK and dV and leaves dQ alone;
* closed forms: identical keys give dQ = 0; constant values give dQ = dK = 0;
  identical keys and constant values give dV_j = mean_i dO_i; a single key gives
  dV = dO; Delta equals sum_d dO O with O from the forward oracle;
* a library cross-check: torch float64 autograd on the CPU.
Planted mistakes (the Delta term dropped, the scale left out of dK, dQ and dK
swapped) must fail the finite-difference pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as ob

RNG = np.random.default_rng(20261202)


def rand(*shape):
    return RNG.standard_normal(shape)


def loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(o * do))


def fd_errors(q, k, v, do, scale, causal, eps=1e-6):
    """Relative error of <grad, E> against a central difference, for each input."""
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    errs = {}
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        e = rand(*x.shape)
        args = {"q": q, "k": k, "v": v}
        args[name] = x + eps * e
        up = loss(args["q"], args["k"], args["v"], do, scale, causal)
        args[name] = x - eps * e
        dn = loss(args["q"], args["k"], args["v"], do, scale, causal)
        fd = (up - dn) / (2 * eps)
        an = float(np.sum(g * e))
        errs[name] = abs(fd - an) / max(1e-12, abs(fd) + abs(an))
    return errs


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,D", [(1, 2), (2, 3), (5, 4), (7, 3)])
def test_finite_differences(causal, N, D):
    q, k, v, do = rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D)
    errs = fd_errors(q, k, v, do, 0.7, causal)
    assert max(errs.values()) < 1e-7, errs


def test_finite_differences_more_keys_than_queries():
    q, k, v, do = rand(1, 1, 3, 4), rand(1, 1, 6, 4), rand(1, 1, 6, 4), rand(1, 1, 3, 4)
    errs = fd_errors(q, k, v, do, 0.5, False)
    assert max(errs.values()) < 1e-7, errs


@pytest.mark.parametrize("mistake", ["no_delta", "unscaled_dk", "swap_dq_dk"])
def test_planted_mistakes_fail_finite_differences(monkeypatch, mistake):
    good = ob._backward_rows

    def broken(qh, kh, vh, doh, scale, causal, r0, r1):
        dq, dk, dv, delta = good(qh, kh, vh, doh, scale, causal, r0, r1)
        if mistake == "no_delta":  # dS = P dP, the Jacobian's second term dropped
            q = qh[r0:r1]
            S = scale * (q @ kh.T)
            if causal:
                S = np.where(np.arange(kh.shape[0])[None, :] <= np.arange(r0, r1)[:, None], S,
                             -math.inf)
            P, _, _ = oracle.safe_softmax_rows(S)
            dS = P * (doh[r0:r1] @ vh.T)
            dq, dk = scale * (dS @ kh), scale * (dS.T @ q)
        elif mistake == "unscaled_dk":
            dk = dk / scale
        else:
            dq, dk = dk[r0:r1], np.pad(dq, ((0, dk.shape[0] - (r1 - r0)), (0, 0)))
        return dq, dk, dv, delta

    monkeypatch.setattr(ob, "_backward_rows", broken)
    q, k, v, do = rand(1, 1, 5, 4), rand(1, 1, 5, 4), rand(1, 1, 5, 4), rand(1, 1, 5, 4)
    errs = fd_errors(q, k, v, do, 0.7, False)
    assert max(errs.values()) > 1e-3, errs


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    q, k, v, do = rand(2, 2, 64, 16), rand(2, 2, 64, 16), rand(2, 2, 64, 16), rand(2, 2, 64, 16)
    _, dk, _, _ = oracle.attention_backward(q, k, v, do, 0.25, causal, row_block=16)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(dk))) * 64


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_zero_dq(causal):
    N, D = 33, 8
    q, v, do = rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D)
    k = np.broadcast_to(rand(D), (1, 1, N, D)).copy()
    dq, _, _, _ = oracle.attention_backward(q, k, v, do, 0.3, causal)
    assert np.max(np.abs(dq)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_zero_dq_dk(causal):
    N, D = 29, 8
    q, k, do = rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D)
    v = np.broadcast_to(rand(D), (1, 1, N, D)).copy()
    dq, dk, _, _ = oracle.attention_backward(q, k, v, do, 0.3, causal)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


def test_identical_keys_constant_values_closed_form_dv():
    N, D = 17, 8
    q, do = rand(1, 1, N, D), rand(1, 1, N, D)
    k = np.broadcast_to(rand(D), (1, 1, N, D)).copy()
    v = np.broadcast_to(rand(D), (1, 1, N, D)).copy()
    _, _, dv, _ = oracle.attention_backward(q, k, v, do, 0.3, False)
    np.testing.assert_allclose(dv[0, 0], np.broadcast_to(do[0, 0].mean(0), (N, D)), atol=1e-13)
    # causal: key j is seen by rows i >= j, each with weight 1 / (i + 1)
    _, _, dvc, _ = oracle.attention_backward(q, k, v, do, 0.3, True)
    w = 1.0 / np.arange(1, N + 1)
    ref = np.array([(w[j:, None] * do[0, 0, j:]).sum(0) for j in range(N)])
    np.testing.assert_allclose(dvc[0, 0], ref, atol=1e-13)


def test_single_key():
    q, k, v, do = rand(2, 3, 1, 8), rand(2, 3, 1, 8), rand(2, 3, 1, 8), rand(2, 3, 1, 8)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.9, False)
    np.testing.assert_allclose(dv, do, atol=1e-15)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15


def test_permuting_keys_permutes_their_gradients():
    N, D = 20, 8
    q, k, v, do = rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, N, D)
    perm = RNG.permutation(N)
    a = oracle.attention_backward(q, k, v, do, 0.4, False)
    b = oracle.attention_backward(q, k[:, :, perm], v[:, :, perm], do, 0.4, False)
    np.testing.assert_allclose(b[0], a[0], atol=1e-13)
    np.testing.assert_allclose(b[1], a[1][:, :, perm], atol=1e-13)
    np.testing.assert_allclose(b[2], a[2][:, :, perm], atol=1e-13)


def test_linear_in_upstream_gradient():
    N, D = 12, 8
    q, k, v = rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D)
    d1, d2 = rand(1, 2, N, D), rand(1, 2, N, D)
    g1 = oracle.attention_backward(q, k, v, d1, 0.4, True)
    g2 = oracle.attention_backward(q, k, v, d2, 0.4, True)
    g12 = oracle.attention_backward(q, k, v, d1 + 2 * d2, 0.4, True)
    for a, b, c in zip(g1[:3], g2[:3], g12[:3]):
        np.testing.assert_allclose(c, a + 2 * b, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_delta_equals_rowsum_do_times_o(causal):
    q, k, v, do = rand(1, 2, 40, 8), rand(1, 2, 40, 8), rand(1, 2, 40, 8), rand(1, 2, 40, 8)
    o, _ = oracle.attention(q, k, v, 0.3, causal)
    _, _, _, delta = oracle.attention_backward(q, k, v, do, 0.3, causal, row_block=7)
    np.testing.assert_allclose(delta, np.sum(do * o, axis=-1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    N, D = 48, 16
    q, k, v, do = rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, N, D)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    S = 0.2 * tq @ tk.transpose(-1, -2)
    if causal:
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(S, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.2, causal, row_block=10)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_the_full_backward(causal):
    """The row-sampled dQ (used at sizes the full oracle cannot hold) is the full
    backward's dQ on those rows: the same routine, one row at a time."""
    g = torch.Generator().manual_seed(321)
    q, k, v, do = (torch.randn(2, 2, 37, 16, generator=g, dtype=torch.float64) for _ in range(4))
    dq = oracle.attention_backward(q, k, v, do, 0.3, causal)[0]
    rows = [(0, 0, 0), (0, 1, 36), (1, 0, 17), (1, 1, 5), (1, 1, 36)]
    got = oracle.attention_backward_dq_rows(q, k, v, do, 0.3, causal, rows)
    want = np.stack([dq[b, h, i] for b, h, i in rows])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_causal_tail_block_gives_the_last_keys_whole_gradients():
    """Under the causal mask the last r keys are seen only by the last r queries, so the
    row block [N - r, N) alone gives their complete dK and dV (as in the full backward)."""
    g = torch.Generator().manual_seed(654)
    q, k, v, do = (torch.randn(1, 2, 40, 8, generator=g, dtype=torch.float64) for _ in range(4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5, True)
    gq, gk, gv = oracle.attention_backward_row_block(q, k, v, do, 0.5, True, 0, 1, 28, 40)
    np.testing.assert_allclose(gq, dq[0, 1, 28:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gk[28:], dk[0, 1, 28:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gv[28:], dv[0, 1, 28:], rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(gk[:28] - dk[0, 1, :28])) > 1e-3  # earlier keys need earlier rows
