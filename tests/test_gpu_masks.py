"""Parity of the mask variants of the forward (fa_forward_ext, through the C ABI) with
the fp64 oracle: sliding windows and packed variable-length batches.

Tolerances as for the dense forward: max |O - O_ref| <= 2e-2 absolute (bfloat16
inputs), max |lse - lse_ref| <= 1e-3, over every row the call is defined to write.
Outputs start as NaN, so a row the kernel misses fails the finiteness check, and rows
the call must not write are checked to be still NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import ORACLE_WORKERS, one_blas_thread
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import WORKLOADS, make_inputs, random_tensor

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3
BIG = 2**31 - 1


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    fa.load()
    yield
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)


def run_ext(q, k, v, scale, causal, wl=-1, wr=-1, cu=None, max_seqlen=0):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    fa.fa_forward_ext(qd, kd, vd, o, lse, scale, causal, wl, wr, cud, max_seqlen)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, o_ref, lse_ref, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output (unwritten rows?)"
    # a row that sees no key has lse = -inf on both sides
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: -inf pattern"
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite lse"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    say(f"{what}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
    assert err_o <= TOL_O, f"{what}: max|dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max|dlse| = {err_l}"


WINDOWS = [(-1, -1), (0, 0), (31, 31), (64, -1), (-1, 64), (100, 37), (255, 0), (256, 300),
           (1000, 1000), (5, BIG), (BIG, 3)]


# ------------------------------------------------------------------ sliding windows
@pytest.mark.parametrize("window", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 333, 700])
def test_window(N, D, causal, window):
    wl, wr = window
    seed = 7 * N + D + 3 * int(causal) + 11 * WINDOWS.index(window)
    q, k, v = (random_tensor((2, 2, N, D), seed + i, torch.bfloat16) for i in range(3))
    scale = 1.0 / math.sqrt(D)
    say(f"window N={N} D={D} causal={causal} wl={wl} wr={wr}")
    o, lse = run_ext(q, k, v, scale, causal, wl, wr)
    o_ref, lse_ref = oracle.attention_window(q, k, v, scale, causal, wl, wr)
    check(o, lse, o_ref, lse_ref, f"window N={N} D={D} causal={causal} ({wl},{wr})")


@pytest.mark.parametrize("window", [(40, 0), (300, 17), (513, -1)])
def test_window_large_scores(window):
    """Scores in the tens (q, k ~ N(0, 9)): the reference maximum is replaced inside and
    at the edges of the window, including right after fully masked blocks."""
    wl, wr = window
    q, k = (random_tensor((1, 3, 900, 128), 300 + i, torch.bfloat16, sigma=3.0) for i in range(2))
    v = random_tensor((1, 3, 900, 128), 302, torch.bfloat16)
    for causal in (False, True):
        o, lse = run_ext(q, k, v, 1 / math.sqrt(128), causal, wl, wr)
        o_ref, lse_ref = oracle.attention_window(q, k, v, 1 / math.sqrt(128), causal, wl, wr)
        check(o, lse, o_ref, lse_ref, f"large scores causal={causal} ({wl},{wr})")


def test_diagonal_window_returns_values():
    """window (0, 0): every row sees only its own key, so its one weight is exactly 1,
    O = v_i exactly and lse = scale q_i . k_i."""
    N, D = 517, 128
    q, k, v = (random_tensor((1, 2, N, D), 320 + i, torch.bfloat16) for i in range(3))
    o, lse = run_ext(q, k, v, 0.1, False, 0, 0)
    assert np.array_equal(o, v.double().numpy())
    s = 0.1 * (q.double() * k.double()).sum(-1).numpy()
    assert np.max(np.abs(lse - s)) <= 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_ext_without_masks_matches_forward_bitwise(causal):
    q, k, v = (random_tensor((2, 2, 777, 64), 330 + i, torch.bfloat16) for i in range(3))
    o1, l1 = run_ext(q, k, v, 0.125, causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o2, l2 = fa.forward(qd, kd, vd, 0.125, causal)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o2.cpu().double().numpy())
    assert np.array_equal(l1, l2.cpu().double().numpy())


# ------------------------------------------------------------------ packed sequences
LENS = [0, 1, 31, 64, 65, 300, 0, 513, 2, 257]


@pytest.mark.parametrize("window", [(-1, -1), (50, 50), (128, 0)], ids=["nowin", "w50", "w128_0"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen(D, causal, window):
    wl, wr = window
    H, extra = 3, 9  # rows past the last sequence: no call may write them
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    total = int(cu[-1]) + extra
    seed = 400 + D + int(causal) + 5 * wl
    q, k, v = (random_tensor((H, total, D), seed + i, torch.bfloat16) for i in range(3))
    scale = 1.0 / math.sqrt(D)
    say(f"varlen D={D} causal={causal} wl={wl} wr={wr}")
    o, lse = run_ext(q, k, v, scale, causal, wl, wr, cu=cu.tolist(), max_seqlen=max(LENS))
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, scale, causal, wl, wr)
    n = int(cu[-1])
    check(o[:, :n], lse[:, :n], o_ref[:, :n], lse_ref[:, :n], f"varlen D={D} causal={causal}")
    assert np.all(np.isnan(o[:, n:])) and np.all(np.isnan(lse[:, n:])), "rows past cu[-1] written"


def test_varlen_equals_separate_dense_calls():
    """Every packed sequence gives exactly what a dense call on it alone gives."""
    lens = [100, 257, 1, 600]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = (random_tensor((2, int(cu[-1]), 128), 450 + i, torch.bfloat16) for i in range(3))
    o, lse = run_ext(q, k, v, 0.09, True, cu=cu.tolist(), max_seqlen=max(lens))
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        od, ld = run_ext(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.09, True)
        assert np.array_equal(o[:, a:b], od[0]) and np.array_equal(lse[:, a:b], ld[0]), s


def test_varlen_max_seqlen_caps_sequences():
    """A sequence longer than max_seqlen is attention over its first max_seqlen rows;
    its later rows are not written."""
    lens, cap = [40, 700, 300], 320
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = (random_tensor((2, int(cu[-1]), 64), 460 + i, torch.bfloat16) for i in range(3))
    o, lse = run_ext(q, k, v, 0.125, False, cu=cu.tolist(), max_seqlen=cap)
    capped = np.array([0, 40, 40 + cap, 40 + cap + 300], dtype=np.int32)
    keep = np.r_[0:40, 40:40 + cap, 740:1040]
    o_ref, lse_ref = oracle.attention_varlen(q[:, keep], k[:, keep], v[:, keep], capped, 0.125)
    check(o[:, keep], lse[:, keep], o_ref, lse_ref, "max_seqlen cap")
    assert np.all(np.isnan(o[:, 40 + cap:740])), "rows past max_seqlen written"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_inconsistent_offsets_are_clamped(causal):
    """Offsets are clamped on the device (a = clamp(cu[s], 0, N), b = clamp(cu[s+1], a,
    N)), so decreasing, negative or oversized entries still define sequences inside the
    tensors: nothing is read or written outside them (guard rows around o and lse stay
    untouched) and each clamped sequence is attention on its own rows. With cu = [0, 120,
    60, 250, 400] the sequences are [0, 120), [120, 120), [60, 250) and [250, 400): rows
    60-119 belong to two sequences, whose stores may interleave: each of their elements
    holds one of the two results."""
    D, total, pad = 128, 400, 64
    q, k, v = (random_tensor((1, total, D), 480 + i + 3 * int(causal), torch.bfloat16)
               for i in range(3))
    for cu, seqs in (([0, 120, 60, 250, 400], [(0, 120), (60, 250), (250, 400)]),
                     ([-5, 100, 5000], [(0, 100), (100, total)])):
        o_big = torch.full((1, pad + total + pad, D), float("nan"), device="cuda")
        l_big = torch.full((1, pad + total + pad), float("nan"), device="cuda")
        o, lse = o_big[:, pad:pad + total], l_big[:, pad:pad + total]
        cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
        fa.fa_forward_ext(q.cuda(), k.cuda(), v.cuda(), o, lse, 0.1, causal, -1, -1, cud, total)
        torch.cuda.synchronize()
        say(f"clamped offsets {cu} causal={causal}")
        assert bool(torch.isnan(o_big[:, :pad]).all() and torch.isnan(o_big[:, pad + total:]).all())
        assert bool(torch.isnan(l_big[:, :pad]).all() and torch.isnan(l_big[:, pad + total:]).all())
        got_o, got_l = o.cpu().double().numpy()[0], lse.cpu().double().numpy()[0]
        refs = {}
        for a, b in seqs:
            ro, rl = oracle.attention(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.1, causal)
            refs[(a, b)] = (ro[0, 0], rl[0, 0])
        for i in range(total):
            owners = [(a, b) for a, b in seqs if a <= i < b]
            assert owners, i
            # two sequences' stores of one row may interleave: every element must be
            # one of its owners' values
            d_o = np.min([np.abs(got_o[i] - refs[s][0][i - s[0]]) for s in owners], axis=0)
            d_l = min(abs(got_l[i] - refs[s][1][i - s[0]]) for s in owners)
            assert np.max(d_o) <= TOL_O and d_l <= TOL_LSE, f"row {i}, sequences {owners}"


# ------------------------------------------------------------------ full size
@pytest.mark.timeout(900)
@pytest.mark.parametrize("window", [1024, 4096])
def test_window_full_size_all_heads(window):
    """The large-score workload's shape (B=2, H=32, N=8192, D=128), causal with the
    benchmark's 1024- and 4096-key windows: every row of every head against the oracle."""
    w = WORKLOADS["large_score_causal_d128"]
    q, k, v = make_inputs(w)
    say(f"window {window} at full size")
    o, lse = run_ext(q, k, v, w.scale, True, window, -1)
    with one_blas_thread():
        o_ref, lse_ref = oracle.attention_window(q, k, v, w.scale, True, window, -1,
                                                 row_block=256, workers=ORACLE_WORKERS)
    check(o, lse, o_ref, lse_ref, f"window {window} full size, all heads")


@pytest.mark.timeout(900)
def test_varlen_full_size_all_sequences():
    """The benchmark's packed batch (H=32, D=128, 32 sequences of 64-4032 rows, causal)
    in one launch; every row of every sequence and head against the oracle."""
    from exact_io_aware_22_amd.workloads import packed_inputs

    w = WORKLOADS["varlen_causal_d128"]
    q, k, v, cu = packed_inputs(w)
    say(f"packed batch at full size: {len(w.seqlens)} sequences, {int(cu[-1])} rows")
    o, lse = run_ext(q, k, v, w.scale, True, -1, -1, cu.tolist(), max(w.seqlens))
    with one_blas_thread():
        o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu.numpy(), w.scale, True,
                                                 workers=ORACLE_WORKERS)
    check(o, lse, o_ref, lse_ref, "packed full size, all sequences and heads")
