"""Plain fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The library's device path never
calls it, and it imports nothing from the library: the two share no code.

The pages name the backward pass (recompute rather than store the attention
matrix, keeping only the per-row log-sum-exp) but print no formula for it, so the
gradients here are derived by the chain rule from the forward definition of
section "FlashAttention: Not So Special" (S = scale Q K^T, P = row softmax(S),
O = P V). For a loss L with upstream gradient dO = dL/dO:

* dV = P^T dO, since O = P V;
* dP = dO V^T, for the same reason;
* the row softmax p = softmax(s) has Jacobian dp_j/ds_k = p_j (delta_jk - p_k),
  so dS_ij = P_ij (dP_ij - Delta_i) with Delta_i = sum_j P_ij dP_ij;
* Delta_i also equals sum_d dO_id O_id, because sum_j P_ij dP_ij =
  sum_j P_ij sum_d dO_id V_jd = sum_d dO_id O_id;
* S = scale Q K^T gives dQ = scale dS K and dK = scale dS^T Q.

Masked keys have P_ij = 0, so they receive no gradient and pass none on. Rows
of P are recomputed from the same definition as the forward oracle, one block
of rows at a time: nothing is approximated, and everything is float64.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .fp64 import NEG_INF, _f64, safe_softmax_rows


def _backward_rows(qh, kh, vh, doh, scale, causal, r0, r1):
    """Gradient contributions of query rows [r0, r1) of one head.

    Returns (dQ rows [r1-r0, D], dK part [Nk, D], dV part [Nk, Dv], Delta rows).
    dK and dV are sums over query rows, so row blocks add up.
    """
    q = qh[r0:r1]
    S = scale * (q @ kh.T)                                  # S = scale Q K^T
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(kh.shape[0])[None, :]
        S = np.where(cols <= rows, S, NEG_INF)              # key j visible iff j <= i
    P, _, _ = safe_softmax_rows(S)                          # P = row softmax(S)
    do = doh[r0:r1]
    dV = P.T @ do                                           # dV = P^T dO
    dP = do @ vh.T                                          # dP = dO V^T
    delta = np.sum(P * dP, axis=1)                          # Delta_i = sum_j P_ij dP_ij
    dS = P * (dP - delta[:, None])                          # softmax Jacobian, row by row
    dQ = scale * (dS @ kh)                                  # dQ = scale dS K
    dK = scale * (dS.T @ q)                                 # dK = scale dS^T Q
    return dQ, dK, dV, delta


def attention_backward(q, k, v, do, scale: float, causal: bool = False, row_block: int = 1024,
                       workers: int = 1):
    """Gradients (dQ, dK, dV) of O = softmax(scale Q K^T) V for upstream gradient dO.

    q: [B, H, N, D]; k, v: [B, H, Nk, D]; do: [B, H, N, Dv] (any float dtype, upcast
    exactly to fp64). Returns float64 arrays dq [B, H, N, D], dk [B, H, Nk, D],
    dv [B, H, Nk, Dv] and delta [B, H, N] (sum_d dO O per row).

    Rows of P are materialised a block of at most `row_block` query rows at a
    time; dK and dV accumulate over the blocks. `workers` only spreads heads
    over threads.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    if causal and Nk != N:
        raise ValueError("causal attention here needs as many keys as queries")
    dq = np.zeros_like(q)
    dk = np.zeros((B, H, Nk, D), dtype=np.float64)
    dv = np.zeros((B, H, Nk, v.shape[3]), dtype=np.float64)
    delta = np.zeros((B, H, N), dtype=np.float64)

    def run(bh):
        b, h = bh
        if Nk == 0:
            return
        for r0 in range(0, N, row_block):
            r1 = min(N, r0 + row_block)
            gq, gk, gv, dl = _backward_rows(q[b, h], k[b, h], v[b, h], do[b, h], float(scale),
                                            causal, r0, r1)
            dq[b, h, r0:r1] = gq
            dk[b, h] += gk
            dv[b, h] += gv
            delta[b, h, r0:r1] = dl

    heads = [(b, h) for b in range(B) for h in range(H)]
    if workers > 1 and len(heads) > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, heads))
    else:
        for bh in heads:
            run(bh)
    return dq, dk, dv, delta


def attention_backward_dq_rows(q, k, v, do, scale: float, causal: bool, rows):
    """dQ for a chosen set of query rows only: rows is an iterable of (b, h, i).

    Row i of dQ = scale dS_i K needs only row i of Q and dO and all of K and V (P_i,
    dP_i and Delta_i are all row-local), so each row is computed alone by the same
    row-block routine as attention_backward, with a block of one row. Returns float64
    [len(rows), D].
    """
    rows = list(rows)
    out = np.zeros((len(rows), q.shape[3]), dtype=np.float64)
    head = None
    for n, (b, h, i) in enumerate(rows):
        if head is None or head[0] != (b, h):
            head = ((b, h), _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h]))
        _, qh, kh, vh, doh = head
        gq, _, _, _ = _backward_rows(qh, kh, vh, doh, float(scale), causal, i, i + 1)
        out[n] = gq[0]
    return out


def attention_backward_row_block(q, k, v, do, scale: float, causal: bool, b: int, h: int,
                                 r0: int, r1: int):
    """The gradient contributions of query rows [r0, r1) of head (b, h): dQ of those
    rows [r1-r0, D] and their parts of dK [Nk, D] and dV [Nk, Dv] (float64).

    Under the causal mask key j is seen only by queries i >= j, so for r1 = N the parts
    are the whole dK and dV of keys j >= r0: the last keys' gradients need only the last
    query rows.
    """
    gq, gk, gv, _ = _backward_rows(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]),
                                   _f64(do[b, h]), float(scale), causal, r0, r1)
    return gq, gk, gv
