"""Plain fp64 CPU oracle for exact attention and its (m, d, o) partial states.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The library's device path never
calls it, and it imports nothing from the library: the two share no code.

Everything here is computed in float64 with numpy, in the plainest order the
pages describe. Sources (all from "Learning FlashAttention the Hard Way --
Part 1", cloudrift.ai):

* softmax and safe softmax, and its three passes (max, sum, divide):
  section "Softmax Looks Like It Breaks the Rules";
* attention S = scale * Q K^T, P = row softmax(S), O = P V, and the per-row
  reading of it: section "FlashAttention: Not So Special";
* the state u = (m, d, o) over a block of keys, the injection (s_j, 1, v_j)
  and the single deferred division o / d: section "The State";
* the combine with its case split on the larger maximum: section "The Merge,
  and the Twist";
* the identity (-inf, 0, 0) and the absolute coordinates D = d e^m,
  O = o e^m (so log-sum-exp = m + ln d): section "Why Attention's Combine
  Still Associates";
* the base-2 twist (sigma = s log2 e, exponentials in base 2): section
  "Alternative Twist: Base 2".

The softmax scale multiplies Q K^T; the pages say a scale is applied (base-2
section) without printing where, and the plainest reading is the one used here.
Causal masking keeps key j visible to query i iff j <= i (queries and keys
share positions). A row whose keys are all masked is the identity state:
output 0, log-sum-exp -inf.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

NEG_INF = -math.inf
LOG2E = 1.0 / math.log(2.0)


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (accepts numpy arrays, or CPU torch tensors of any float dtype)."""
    if hasattr(x, "detach"):  # a torch tensor: upcast in torch first so bf16 converts exactly
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------- softmax
def safe_softmax_rows(S: np.ndarray):
    """Safe softmax of every row of S, in the three passes the pages list.

    Pass 1: m = max_j s_j.  Pass 2: d = sum_j e^{s_j - m}.  Pass 3: p_i = e^{s_i - m} / d.
    (section "Softmax Looks Like It Breaks the Rules").  A row of all -inf is the
    identity state: m = -inf, d = 0, p = 0.
    Returns (P, m, d).
    """
    S = np.asarray(S, dtype=np.float64)
    m = S.max(axis=-1)
    m_ref = np.where(np.isneginf(m), 0.0, m)
    E = np.exp(S - m_ref[..., None])
    d = E.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = np.where(d[..., None] > 0.0, E / np.where(d > 0.0, d, 1.0)[..., None], 0.0)
    return P, m, d


def logsumexp_from_state(m, d):
    """ln sum_j e^{s_j} = m + ln d: the absolute-coordinate denominator D = d e^m
    (section "Why Attention's Combine Still Associates").  Identity -> -inf."""
    m = np.asarray(m, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = m + np.log(d)
    return np.where(d > 0.0, out, NEG_INF)


# --------------------------------------------------------------------------- attention
def _attention_rows(qh, kh, vh, scale, causal, r0, r1):
    S = scale * (qh[r0:r1] @ kh.T)                       # S = scale * Q K^T, materialised
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(kh.shape[0])[None, :]
        S = np.where(cols <= rows, S, NEG_INF)          # key j visible iff j <= i
    P, m, d = safe_softmax_rows(S)                       # P = row softmax(S)
    return P @ vh, logsumexp_from_state(m, d)            # O = P V ; lse = m + ln d


def attention(q, k, v, scale: float, causal: bool = False, row_block: int = 1024,
              workers: int = 1):
    """Exact attention O = softmax(scale * Q K^T) V and per-row log-sum-exp.

    q: [B, H, N, D]; k, v: [B, H, Nk, D] (any float dtype; upcast exactly to fp64).
    Returns (O [B, H, N, D] float64, lse [B, H, N] float64, natural log).

    The score and probability matrices are materialised (a block of at most
    `row_block` rows at a time), the standard schedule that the tiled method
    is shown equal to (section "FlashAttention: Not So Special").  `workers`
    only spreads independent (b, h, row-block) units over threads.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    if causal and Nk != N:
        raise ValueError("causal attention here needs as many keys as queries")
    o = np.zeros((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, N), NEG_INF, dtype=np.float64)
    units = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, N, row_block)]

    def run(unit):
        b, h, r0 = unit
        r1 = min(N, r0 + row_block)
        if Nk == 0:
            return
        ob, lb = _attention_rows(q[b, h], k[b, h], v[b, h], float(scale), causal, r0, r1)
        o[b, h, r0:r1] = ob
        lse[b, h, r0:r1] = lb

    if workers > 1 and len(units) > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, units))
    else:
        for u in units:
            run(u)
    return o, lse


def attention_base2(q, k, v, scale: float, causal: bool = False):
    """The same attention with every exponential taken in base 2.

    sigma_j = s_j * log2(e); m = max sigma; d = sum 2^{sigma_j - m};
    weight_j = 2^{sigma_j - m} / d; lse = (m + log2 d) / log2(e)
    (section "Alternative Twist: Base 2").  Row-at-a-time, fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.full((B, H, N), NEG_INF)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                s = float(scale) * (k[b, h] @ q[b, h, i])
                if causal:
                    s = s[: i + 1]
                sigma = s * LOG2E
                m = sigma.max()
                w = np.exp2(sigma - m)
                d = w.sum()
                o[b, h, i] = (w @ v[b, h, : len(w)]) / d
                lse[b, h, i] = (m + math.log2(d)) / LOG2E
    return o, lse


# --------------------------------------------------------------------------- the (m, d, o) state
def identity_state(D: int):
    """The neutral element (-inf, 0, 0) (section "Why Attention's Combine Still Associates")."""
    return (NEG_INF, 0.0, np.zeros(D))


def inject(s_j: float, v_j) -> tuple:
    """One key/value pair enters as (s_j, 1, v_j) (section "The State")."""
    return (float(s_j), 1.0, np.array(v_j, dtype=np.float64))


def combine(ua, ub):
    """u_a (+) u_b: keep the larger maximum and shrink the other side by
    e^{(smaller max) - (larger max)} (section "The Merge, and the Twist").

    Identity states (m = -inf) pass the other operand through unchanged, which
    is what the formally adjoined identity means (section "Welford, the Easy Way").
    """
    ma, da, oa = ua
    mb, db, ob = ub
    if ma >= mb:
        if mb == NEG_INF:
            return (ma, da, np.array(oa, dtype=np.float64))
        f = math.exp(mb - ma)
        return (ma, da + db * f, oa + ob * f)
    f = math.exp(ma - mb)
    return (mb, db + da * f, ob + oa * f)


def block_state(s, V):
    """The state of one block of keys, straight from its definition
    m = max_j s_j, d = sum_j e^{s_j - m}, o = sum_j e^{s_j - m} v_j
    (section "The State").  An empty or fully masked block is the identity."""
    s = np.asarray(s, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    D = V.shape[-1]
    if s.size == 0 or np.all(np.isneginf(s)):
        return identity_state(D)
    m = float(s.max())
    w = np.exp(s - m)
    return (m, float(w.sum()), w @ V)


def readout(u):
    """Output row o / d and log-sum-exp m + ln d: the one deferred division
    (section "The State").  The identity reads out as (0, -inf)."""
    m, d, o = u
    if d == 0.0:
        return np.zeros_like(np.asarray(o, dtype=np.float64)), NEG_INF
    return np.asarray(o, dtype=np.float64) / d, m + math.log(d)


# --------------------------------------------------------------------------- split-KV decode
def split_bounds(L: int, splits: int):
    """Chunk s covers keys [s*c, min(L, (s+1)*c)) with c = ceil(L / splits); a chunk
    past the end is empty."""
    c = -(-L // splits) if L > 0 else 0
    return [(min(L, s * c), min(L, (s + 1) * c)) for s in range(splits)]


def decode_partials(q, k, v, scale: float, splits: int):
    """Per-chunk partial states for single-query attention (split-K: separate
    blocks own chunks and write partials; section "Associativity is All You
    Need", and split-KV in section "Why Attention's Combine Still Associates").

    q: [B, H, 1, D] (or [B, H, D]); k, v: [B, H, L, D].
    Returns m [B*H, splits], d [B*H, splits], o [B*H, splits, D] (fp64); m is in
    natural-log units of the scaled score, o is unnormalised.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, D = k.shape
    q = q.reshape(B, H, D)
    m = np.full((B * H, splits), NEG_INF)
    d = np.zeros((B * H, splits))
    o = np.zeros((B * H, splits, v.shape[3]))
    bounds = split_bounds(L, splits)
    for b in range(B):
        for h in range(H):
            s_all = float(scale) * (k[b, h] @ q[b, h])
            for sp, (j0, j1) in enumerate(bounds):
                ms, ds, os_ = block_state(s_all[j0:j1], v[b, h, j0:j1])
                m[b * H + h, sp], d[b * H + h, sp], o[b * H + h, sp] = ms, ds, os_
    return m, d, o


def combine_partials(m, d, o_part):
    """Fold each row's partial states left to right with (+), then read out.

    m, d: [rows, splits]; o_part: [rows, splits, D].  Returns (o [rows, D], lse [rows]).
    """
    m, d, o_part = _f64(m), _f64(d), _f64(o_part)
    rows, splits = m.shape
    D = o_part.shape[2]
    out = np.zeros((rows, D))
    lse = np.full(rows, NEG_INF)
    for r in range(rows):
        u = identity_state(D)
        for s in range(splits):
            u = combine(u, (float(m[r, s]), float(d[r, s]), o_part[r, s]))
        out[r], lse[r] = readout(u)
    return out, lse


def attention_selected_rows(q, k, v, scale: float, causal: bool, rows):
    """Attention for a chosen set of query rows only, one row at a time.

    rows: iterable of (b, h, i).  Returns (O [len(rows), D], lse [len(rows)]).
    Row i of O depends only on row i of Q and all of K and V (section
    "FlashAttention: Not So Special"), so any row can be computed alone.
    """
    rows = list(rows)
    D = v.shape[3]
    out = np.zeros((len(rows), D))
    lse = np.full(len(rows), NEG_INF)
    for n, (b, h, i) in enumerate(rows):
        kb = _f64(k[b, h])
        vb = _f64(v[b, h])
        qi = _f64(q[b, h, i])
        if causal:
            kb, vb = kb[: i + 1], vb[: i + 1]
        if kb.shape[0] == 0:
            continue
        S = float(scale) * (qi[None, :] @ kb.T)
        P, m, d = safe_softmax_rows(S)
        out[n] = (P @ vb)[0]
        lse[n] = logsumexp_from_state(m, d)[0]
    return out, lse
