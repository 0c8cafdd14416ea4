"""Parity of the backward pass (fa_backward, through the C ABI) with the fp64 oracle.

The GPU gradients are computed from the GPU forward's o and lse, as a training step
would; the oracle computes everything from the inputs in fp64. Tolerance, normwise
per tensor: max |g - g_ref| <= TOL * max(1, max |g_ref|), with TOL = 1e-2 for
bfloat16 inputs (P and dS are rounded to bfloat16, unit roundoff 2^-8, before the
products that consume them; the margin covers float32 accumulation over N terms and
the forward's own error reaching Delta) and 1e-4 for float32 inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import one_blas_thread, parallel_map
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import WORKLOADS, make_inputs, random_tensor

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-4}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    fa.load()
    yield
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)


def run_backward(q, k, v, do, scale, causal):
    qd, kd, vd, dd = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, scale, causal)
    B, H, N, D = q.shape
    delta = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    grads = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda")
             for _ in range(3)]
    fa.fa_backward(qd, kd, vd, o, lse, dd, delta, *grads, scale, causal)
    torch.cuda.synchronize()
    return [g.cpu().double().numpy() for g in grads]


def check(got, ref, dtype, what):
    worst = 0.0
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite output"
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        lim = TOL[dtype] * max(1.0, float(np.max(np.abs(r))) if r.size else 1.0)
        say(f"{what} {name}: max|err| {err:.3e} (limit {lim:.3e})")
        assert err <= lim, f"{what} {name}: {err} > {lim}"
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1, 31, 64, 65, 127, 200, 333])
def test_backward_sizes(dtype, D, causal, N):
    seed = 1000 + N + 7 * D + (1 if causal else 0)
    q, k, v, do = (random_tensor((1, 2, N, D), seed + i, dtype) for i in range(4))
    scale = 1 / math.sqrt(D)
    say(f"backward N={N} D={D} causal={causal} {dtype}")
    got = run_backward(q, k, v, do, scale, causal)
    ref = oracle.attention_backward(q, k, v, do, scale, causal)[:3]
    check(got, ref, dtype, f"N={N} D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1537, 2049])
def test_backward_sizes_past_1024(D, causal, N):
    """Several 256-row query and key tiles of the two kernels, each length one row past a
    64-row staging tile (the ragged last tile stages row N - 1 into its missing rows)."""
    seed = 7000 + N + 7 * D + (1 if causal else 0)
    q, k, v, do = (random_tensor((1, 2, N, D), seed + i, torch.bfloat16) for i in range(4))
    scale = 1 / math.sqrt(D)
    say(f"backward N={N} D={D} causal={causal} bf16")
    got = run_backward(q, k, v, do, scale, causal)
    ref = oracle.attention_backward(q, k, v, do, scale, causal)[:3]
    check(got, ref, torch.bfloat16, f"N={N} D={D} causal={causal}")


def test_backward_large_scores_and_batches():
    """Several heads and batches, scores in the tens (q, k ~ N(0, 9))."""
    q, k = (random_tensor((2, 3, 300, 128), 40 + i, torch.bfloat16, sigma=3.0) for i in range(2))
    v, do = (random_tensor((2, 3, 300, 128), 42 + i, torch.bfloat16) for i in range(2))
    for causal in (False, True):
        got = run_backward(q, k, v, do, 1 / math.sqrt(128), causal)
        ref = oracle.attention_backward(q, k, v, do, 1 / math.sqrt(128), causal)[:3]
        check(got, ref, torch.bfloat16, f"large scores causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_zero_dq_dk(causal):
    N, D = 190, 128
    q, k, do = (random_tensor((1, 2, N, D), 50 + i, torch.bfloat16) for i in range(3))
    v = random_tensor((D,), 53, torch.bfloat16).expand(1, 2, N, D).contiguous()
    dq, dk, dv = run_backward(q, k, v, do, 1 / math.sqrt(D), causal)
    # dS = P (dP - Delta) vanishes exactly; what remains is rounding of Delta and dP
    assert np.max(np.abs(dq)) < 2e-3 and np.max(np.abs(dk)) < 2e-3, (np.max(np.abs(dq)),
                                                                      np.max(np.abs(dk)))


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_zero_dq(causal):
    N, D = 150, 64
    q, v, do = (random_tensor((1, 1, N, D), 60 + i, torch.bfloat16) for i in range(3))
    k = random_tensor((D,), 63, torch.bfloat16).expand(1, 1, N, D).contiguous()
    dq, _, _ = run_backward(q, k, v, do, 0.125, causal)
    assert np.max(np.abs(dq)) < 5e-3, np.max(np.abs(dq))


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    N, D = 520, 128
    q, k, v, do = (random_tensor((1, 2, N, D), 70 + i, torch.bfloat16) for i in range(4))
    _, dk, _ = run_backward(q, k, v, do, 1 / math.sqrt(D), causal)
    s = np.abs(dk.sum(axis=2)).max()
    assert s <= 2e-2 * np.abs(dk).max() * math.sqrt(N), s


@pytest.mark.timeout(900)
def test_backward_full_size_all_heads():
    """The large-score workload at full size (B=2, H=32, N=8192, D=128, causal), run as
    the benchmark runs it; every head's dq, dk and dv against the oracle."""
    w = WORKLOADS["large_score_causal_d128"]
    q, k, v = make_inputs(w)
    do = random_tensor(tuple(q.shape), 99, torch.bfloat16)
    got = run_backward(q, k, v, do, w.scale, w.causal)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return oracle.attention_backward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                         v[b:b + 1, h:h + 1], do[b:b + 1, h:h + 1], w.scale,
                                         w.causal, row_block=512, workers=1)[:3]

    with one_blas_thread():
        refs = parallel_map(one, heads)
    for (b, h), ref in zip(heads, refs):
        check([g[b:b + 1, h:h + 1] for g in got], ref, torch.bfloat16,
              f"full size head ({b},{h})")
