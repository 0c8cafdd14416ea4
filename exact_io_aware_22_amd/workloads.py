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
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(D), rounded to float32 (the value the library receives)."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    def flops(self) -> float:
        """Attention flops, 4*B*H*N*L*D, halved for causal (the usual convention)."""
        f = 4.0 * self.B * self.H * self.N * self.L * self.D
        return f / 2.0 if self.causal else f


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
    ]
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


def random_tensor(shape, seed: int, dtype=torch.bfloat16, sigma: float = 1.0) -> torch.Tensor:
    """A seeded N(0, sigma^2) tensor of any shape (for edge-case tests)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        x = x * torch.tensor(sigma, dtype=torch.float32)
    return x.to(dtype)
