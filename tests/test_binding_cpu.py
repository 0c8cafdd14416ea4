"""The Python binding validates every tensor before it hands raw pointers to libfa.so.

The C ABI receives pointers and sizes only, so a tensor of the wrong shape, dtype or
device would be read or written out of bounds on the GPU, or read with the wrong
element type. Each C-named wrapper must reject such a call with TypeError or
ValueError before the library is touched. These tests run on the CPU: shape and
dtype mistakes are caught before the device check, and well-formed CPU tensors are
refused by the device check.
"""
import pytest
import torch

from exact_io_aware_22_amd import fa

BF, F32 = torch.bfloat16, torch.float32


def z(*shape, dtype=F32):
    return torch.zeros(*shape, dtype=dtype)


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    """Any call that reached the library would fail this test."""
    def boom():
        raise AssertionError("validation let the call reach the library")
    monkeypatch.setattr(fa, "load", boom)


def fwd_args(B=1, H=2, N=8, D=64, dtype=BF):
    return dict(q=z(B, H, N, D, dtype=dtype), k=z(B, H, N, D, dtype=dtype),
                v=z(B, H, N, D, dtype=dtype), o=z(B, H, N, D), lse=z(B, H, N))


@pytest.mark.parametrize("bad,exc", [
    (dict(k=z(1, 2, 9, 64, dtype=BF)), ValueError),        # k longer than q
    (dict(v=z(1, 2, 8, 128, dtype=BF)), ValueError),       # v of another head dim
    (dict(k=z(1, 2, 8, 64, dtype=F32)), TypeError),        # q bf16, k fp32
    (dict(o=z(1, 2, 8, 64, dtype=BF)), TypeError),         # o must be fp32
    (dict(o=z(1, 2, 7, 64)), ValueError),                  # undersized o
    (dict(lse=z(1, 2, 8, 1)), ValueError),
    (dict(lse=z(1, 2, 8, dtype=BF)), TypeError),
    (dict(q=z(2, 8, 64, dtype=BF)), ValueError),           # q not 4-D
    (dict(q=z(1, 2, 8, 64, dtype=torch.float16), k=z(1, 2, 8, 64, dtype=torch.float16),
          v=z(1, 2, 8, 64, dtype=torch.float16)), TypeError),
])
def test_forward_rejects_mismatched_tensors(bad, exc):
    a = fwd_args()
    a.update(bad)
    with pytest.raises(exc):
        fa.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.125, False)


def test_forward_rejects_host_tensors_and_strided_views():
    a = fwd_args()
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.125, False)
    big = z(1, 2, 8, 128)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_forward(a["q"], a["k"], a["v"], big[..., ::2], a["lse"], 0.125, False)


def test_forward_ext_packed_shapes():
    H, T, D = 2, 10, 64
    q, k, v = (z(H, T, D, dtype=BF) for _ in range(3))
    o, lse = z(H, T, D), z(H, T)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(TypeError):
        fa.fa_forward_ext(q, k, v, o, lse, 0.125, True, cu_seqlens=cu.long(), max_seqlen=6)
    with pytest.raises(ValueError):
        fa.fa_forward_ext(q, k, v, o, z(1, H, T), 0.125, True, cu_seqlens=cu, max_seqlen=6)
    with pytest.raises(ValueError):
        fa.fa_forward_ext(q, k, v, o, lse, 0.125, True, cu_seqlens=cu.view(1, 3), max_seqlen=6)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_forward_ext(q, k, v, o, lse, 0.125, True, cu_seqlens=cu, max_seqlen=6)


def dec_args(B=2, H=3, L=16, D=64, splits=4, dtype=BF):
    return dict(q=z(B, H, 1, D, dtype=dtype), k=z(B, H, L, D, dtype=dtype),
                v=z(B, H, L, D, dtype=dtype), m=z(B * H, splits), d=z(B * H, splits),
                o_part=z(B * H, splits, D))


@pytest.mark.parametrize("bad,exc", [
    (dict(q=z(2, 3, 1, 128, dtype=BF)), ValueError),       # q of another head dim
    (dict(q=z(2, 3, 1, 64, dtype=F32)), TypeError),        # q fp32, k bf16
    (dict(v=z(2, 3, 15, 64, dtype=BF)), ValueError),       # v shorter than k
    (dict(m=z(6, 3)), ValueError),                         # fewer splits than asked
    (dict(d=z(6, 4, dtype=BF)), TypeError),
    (dict(o_part=z(6, 4, 32)), ValueError),
])
def test_decode_partials_rejects_mismatched_tensors(bad, exc):
    a = dec_args()
    a.update(bad)
    with pytest.raises(exc):
        fa.fa_decode_partials(a["q"], a["k"], a["v"], a["m"], a["d"], a["o_part"], 0.125, 4)


def test_decode_partials_rejects_zero_splits_and_host_tensors():
    a = dec_args()
    with pytest.raises(ValueError):
        fa.fa_decode_partials(a["q"], a["k"], a["v"], a["m"], a["d"], a["o_part"], 0.125, 0)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_decode_partials(a["q"], a["k"], a["v"], a["m"], a["d"], a["o_part"], 0.125, 4)


@pytest.mark.parametrize("bad,exc", [
    (dict(m=z(5, 4)), ValueError),
    (dict(d=z(6, 4, dtype=BF)), TypeError),
    (dict(o=z(6, 128)), ValueError),
    (dict(lse=z(6, 1)), ValueError),
    (dict(o_part=z(6, 4, 64, dtype=BF)), TypeError),
])
def test_combine_rejects_mismatched_tensors(bad, exc):
    a = dict(m=z(6, 4), d=z(6, 4), o_part=z(6, 4, 64), o=z(6, 64), lse=z(6))
    a.update(bad)
    with pytest.raises(exc):
        fa.fa_combine_partials(a["m"], a["d"], a["o_part"], a["o"], a["lse"])


def test_backward_rejects_mismatched_tensors():
    B, H, N, D = 1, 2, 8, 64
    good = dict(q=z(B, H, N, D, dtype=BF), k=z(B, H, N, D, dtype=BF), v=z(B, H, N, D, dtype=BF),
                o=z(B, H, N, D), lse=z(B, H, N), dout=z(B, H, N, D, dtype=BF),
                delta=z(B, H, N), dq=z(B, H, N, D), dk=z(B, H, N, D), dv=z(B, H, N, D))
    order = ("q", "k", "v", "o", "lse", "dout", "delta", "dq", "dk", "dv")
    for name, bad, exc in [("dout", z(B, H, N, D), TypeError),
                           ("dk", z(B, H, N, D, dtype=BF), TypeError),
                           ("delta", z(B, H, N - 1), ValueError),
                           ("dv", z(B, H, N, 2 * D), ValueError),
                           ("v", z(B, H, N + 1, D, dtype=BF), ValueError)]:
        a = dict(good)
        a[name] = bad
        with pytest.raises(exc):
            fa.fa_backward(*(a[x] for x in order), 0.125, True)
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_backward(*(good[x] for x in order), 0.125, True)


def test_reductions_and_scans_check_outputs():
    x = z(4, 10)
    with pytest.raises(TypeError):
        fa.fa_softmax_stats(x, z(4, dtype=BF), z(4))
    with pytest.raises(ValueError):
        fa.fa_moments(x, z(3), z(4))
    with pytest.raises(TypeError):
        fa.fa_softmax_stats(z(4, 10, dtype=torch.float16), z(4), z(4))
    with pytest.raises(ValueError):
        fa.fa_moments_scan(x, z(4, 9), z(4, 10))
    with pytest.raises(TypeError):
        fa.fa_softmax_scan(x, z(4, 10, dtype=BF), z(4, 10))
    with pytest.raises(ValueError, match="CUDA"):
        fa.fa_softmax_scan(x, z(4, 10), z(4, 10))
