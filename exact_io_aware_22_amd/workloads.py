"""Seeded synthetic workloads: shapes, seeds and random draws only.

This module holds no attention arithmetic. It is the one piece the device path's
tests, the benchmark and the CPU oracle's callers share: every input both sides
see comes from `make_inputs`, drawn on the CPU with a torch.Generator so that the
values do not depend on the device they later live on.

Recipe (each workload has its own generator and seed): for each of q, k, v in
that order, and for each (b, h) slice in row-major order, draw a float32
standard normal slice of shape [rows, D], multiply it by that tensor's sigma
(in float32) and cast it to the workload's dtype (round to nearest even for
bfloat16). Drawing slice by slice keeps the stream identical however large the
tensor is.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int          # query rows per head (1 for single-token decode)
    L: int          # key/value rows per head
    D: int
    dtype: torch.dtype
    causal: bool
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    splits: int = 0  # split-KV decode only: number of key chunks
    window_left: int = -1   # sliding window: key j visible to query i iff
    window_right: int = -1  # i - window_left <= j <= i + window_right (-1: unbounded)
    seqlens: tuple = ()     # packed batch: sequence lengths (then B = len, N = sum)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(D), rounded to float32 (the value the library receives)."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def masked(self) -> bool:
        return bool(self.seqlens) or self.window_left >= 0 or self.window_right >= 0

    def visible_pairs(self) -> int:
        """(query, key) pairs a row may see, summed over rows and heads."""
        if self.seqlens:
            return self.H * sum(_pairs(n, self.causal, self.window_left, self.window_right)
                                for n in self.seqlens)
        return self.B * self.H * _pairs(self.N, self.causal, self.window_left,
                                        self.window_right)

    def flops(self) -> float:
        """Attention flops: 4*B*H*N*L*D, halved for causal (the usual convention); for a
        window or a packed batch, 4*D per visible (query, key) pair."""
        if self.masked:
            return 4.0 * self.D * self.visible_pairs()
        f = 4.0 * self.B * self.H * self.N * self.L * self.D
        return f / 2.0 if self.causal else f


def _pairs(n: int, causal: bool, wl: int, wr: int) -> int:
    """Number of (i, j) in [0, n)^2 with max(0, i - wl) <= j <= min(n - 1, i + wr)."""
    i = torch.arange(n, dtype=torch.int64)
    lo = torch.clamp(i - wl, min=0) if wl >= 0 else torch.zeros_like(i)
    r = 0 if causal else wr
    hi = torch.clamp(i + r, max=n - 1) if r >= 0 else torch.full_like(i, n - 1)
    return int(torch.clamp(hi - lo + 1, min=0).sum())


def _seqlens(seed: int, count: int, lo: int, hi: int) -> tuple:
    """`count` sequence lengths drawn uniformly from [lo, hi] with a seeded generator."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (count,), generator=gen))


def _catalog():
    bf16, f32 = torch.bfloat16, torch.float32
    w = [
        Workload("single_head_fp32", 1, 1, 256, 256, 64, f32, False, 1,
                 note="single head, fp32, N=256, D=64, non-causal"),
        Workload("batched_prefill_d64", 4, 16, 2048, 2048, 64, bf16, False, 2,
                 note="batched prefill, bf16, N=2048, D=64, non-causal"),
        Workload("batched_prefill_d64_causal", 4, 16, 2048, 2048, 64, bf16, True, 2,
                 note="batched prefill, bf16, N=2048, D=64, causal"),
        Workload("large_score_causal_d128", 2, 32, 8192, 8192, 128, bf16, True, 3,
                 sigma_qk=3.0, note="q, k ~ N(0, 9): raw scores in the tens"),
        Workload("split_kv_decode", 16, 32, 1, 32768, 128, bf16, False, 4, splits=64,
                 note="one query row per head, 64 chunks of 512 keys"),
        Workload("long_context_causal_32768", 1, 16, 32768, 32768, 128, bf16, True, 5,
                 note="long context, N a multiple of every tile"),
        Workload("long_context_causal_32767", 1, 16, 32767, 32767, 128, bf16, True, 5,
                 note="long context, ragged tail"),
        Workload("sliding_window_4096_causal_d128", 2, 32, 8192, 8192, 128, bf16, True, 3,
                 sigma_qk=3.0, window_left=4095,
                 note="the large-score inputs; each query sees itself and 4095 keys before it"),
        Workload("sliding_window_1024_causal_d128", 2, 32, 8192, 8192, 128, bf16, True, 3,
                 sigma_qk=3.0, window_left=1023,
                 note="the large-score inputs; each query sees itself and 1023 keys before it"),
    ]
    lens = _seqlens(6, 32, 64, 4032)
    w.append(Workload("varlen_causal_d128", len(lens), 32, sum(lens), sum(lens), 128, bf16,
                      True, 6, seqlens=lens,
                      note="packed batch of 32 causal sequences, lengths uniform in [64, 4032]"))
    return {x.name: x for x in w}


WORKLOADS = _catalog()


def _draw(gen: torch.Generator, lead: tuple, rows: int, D: int, sigma: float,
          dtype: torch.dtype) -> torch.Tensor:
    out = torch.empty(*lead, rows, D, dtype=dtype)
    flat = out.view(-1, rows, D)
    s = torch.tensor(sigma, dtype=torch.float32)
    for idx in range(flat.shape[0]):
        x = torch.randn(rows, D, generator=gen, dtype=torch.float32)
        if sigma != 1.0:
            x = x * s
        flat[idx] = x.to(dtype)
    return out


def make_inputs(w: Workload | str, B: int | None = None, H: int | None = None,
                N: int | None = None, L: int | None = None):
    """q [B, H, N, D], k and v [B, H, L, D] on the CPU, drawn by the recipe above.

    B, H, N, L override the workload's sizes (smaller cases for tests); the seed
    and distributions stay the workload's.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    if L is None:
        L = N if w.N == w.L else w.L  # self-attention keeps as many keys as queries
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    q = _draw(gen, (B, H), N, w.D, w.sigma_qk, w.dtype)
    k = _draw(gen, (B, H), L, w.D, w.sigma_qk, w.dtype)
    v = _draw(gen, (B, H), L, w.D, w.sigma_v, w.dtype)
    return q, k, v


def packed_inputs(w: Workload | str):
    """A packed batch: q, k, v [H, total, D] (every head's rows drawn by the recipe above,
    head by head) and cu_seqlens [nseq + 1] int32 offsets, all on the CPU."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    total = sum(w.seqlens)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    q = _draw(gen, (w.H,), total, w.D, w.sigma_qk, w.dtype)
    k = _draw(gen, (w.H,), total, w.D, w.sigma_qk, w.dtype)
    v = _draw(gen, (w.H,), total, w.D, w.sigma_v, w.dtype)
    cu = torch.zeros(len(w.seqlens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(w.seqlens, dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, cu


@dataclass(frozen=True)
class RowWorkload:
    """A [rows, n] matrix for the row reductions: offset + sigma * N(0, 1) in float32,
    cast to dtype, drawn 1024 rows at a time from one seeded generator."""
    name: str
    rows: int
    n: int
    dtype: torch.dtype
    seed: int
    sigma: float = 1.0
    offset: float = 0.0
    note: str = field(default="", compare=False)

    def bytes_read(self) -> int:
        return self.rows * self.n * torch.finfo(self.dtype).bits // 8

    def bytes_written(self) -> int:
        return self.rows * 2 * 4  # two float32 outputs per row


ROW_WORKLOADS = {w.name: w for w in [
    RowWorkload("softmax_stats_logits_fp32", 8192, 32768, torch.float32, 7, sigma=8.0,
                note="8192 rows of 32768 float32 logits, N(0, 64): scores in the tens"),
    RowWorkload("moments_activations_bf16", 65536, 8192, torch.bfloat16, 8, sigma=1.0,
                offset=3.0, note="65536 rows of 8192 bf16 activations, 3 + N(0, 1)"),
]}


def make_rows(w: RowWorkload | str, rows: int | None = None) -> torch.Tensor:
    """x [rows, n] on the CPU, by the RowWorkload recipe (the first `rows` rows)."""
    if isinstance(w, str):
        w = ROW_WORKLOADS[w]
    rows = w.rows if rows is None else rows
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    out = torch.empty(rows, w.n, dtype=w.dtype)
    s = torch.tensor(w.sigma, dtype=torch.float32)
    o = torch.tensor(w.offset, dtype=torch.float32)
    for r0 in range(0, rows, 1024):
        r1 = min(rows, r0 + 1024)
        x = torch.randn(r1 - r0, w.n, generator=gen, dtype=torch.float32)
        out[r0:r1] = (x * s + o).to(w.dtype)
    return out


def random_tensor(shape, seed: int, dtype=torch.bfloat16, sigma: float = 1.0) -> torch.Tensor:
    """A seeded N(0, sigma^2) tensor of any shape (for edge-case tests)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        x = x * torch.tensor(sigma, dtype=torch.float32)
    return x.to(dtype)
