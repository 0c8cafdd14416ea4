"""Plain fp64 CPU oracle for attention under sliding-window masks and for packed
variable-length batches.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The library's device path never
calls it, and it imports nothing from the library: the two share no code.

Masked keys enter as the identity of the fold, i.e. they get score -inf and weight 0
("Learning FlashAttention the Hard Way -- Part 1", sections "Associativity is All You
Need" and "Why Attention's Combine Still Associates": padding with the neutral
element changes nothing). A mask variant therefore only changes which keys a row
sees; everything else is the plain attention of section "FlashAttention: Not So
Special", materialised a block of rows at a time.

Window: key j is visible to query i iff i - window_left <= j <= i + window_right,
where a negative bound means unbounded on that side; causal additionally requires
j <= i (it is the window_right = 0 case). Packed batches: sequence s occupies rows
[cu_seqlens[s], cu_seqlens[s+1]) of every head, and its queries see only its keys,
with positions counted from the start of the sequence.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .fp64 import NEG_INF, _f64, logsumexp_from_state, safe_softmax_rows


def visible(rows, cols, causal: bool, window_left: int, window_right: int):
    """Boolean mask [len(rows), len(cols)]: key cols[j] visible to query rows[i]."""
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        ok &= j <= i
    if window_left >= 0:
        ok &= j >= i - window_left
    if window_right >= 0:
        ok &= j <= i + window_right
    return ok


def attention_window(q, k, v, scale: float, causal: bool = False, window_left: int = -1,
                     window_right: int = -1, row_block: int = 1024, workers: int = 1):
    """Exact attention of q [B, H, N, D] against k, v [B, H, N, D] under a window.

    Returns (O [B, H, N, D], lse [B, H, N]) in float64; a row that sees no key is the
    identity (O = 0, lse = -inf). `workers` only spreads the independent
    (b, h, row-block) units over threads.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.full((B, H, N), NEG_INF)
    cols = np.arange(Nk)

    def run(unit):
        b, h, r0 = unit
        r1 = min(N, r0 + row_block)
        if Nk == 0:
            return
        S = scale * (q[b, h, r0:r1] @ k[b, h].T)                    # S = scale Q K^T
        S = np.where(visible(np.arange(r0, r1), cols, causal, window_left,
                             window_right), S, NEG_INF)             # masked -> identity
        P, m, d = safe_softmax_rows(S)
        o[b, h, r0:r1] = P @ v[b, h]
        lse[b, h, r0:r1] = logsumexp_from_state(m, d)

    units = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, N, row_block)]
    if workers > 1 and len(units) > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, units))
    else:
        for u in units:
            run(u)
    return o, lse


def attention_varlen(q, k, v, cu_seqlens, scale: float, causal: bool = False,
                     window_left: int = -1, window_right: int = -1, workers: int = 1):
    """Packed variable-length attention: q, k, v [H, total, D]; cu_seqlens [nseq + 1]
    (nondecreasing, cu_seqlens[0] = 0, cu_seqlens[-1] = total). Every sequence is
    attention on its own rows. Returns (O [H, total, D], lse [H, total]) in float64.
    `workers` is passed on to attention_window (threads over its row blocks)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    H, total, D = q.shape
    o = np.zeros((H, total, v.shape[2]))
    lse = np.full((H, total), NEG_INF)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            continue
        os_, ls_ = attention_window(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], scale,
                                    causal, window_left, window_right, workers=workers)
        o[:, a:b] = os_[0]
        lse[:, a:b] = ls_[0]
    return o, lse
