"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on one MI355X.

Tolerances: max |O - O_ref| <= 2e-2 absolute for bfloat16 inputs and <= 1e-4 for
float32 inputs, max |lse - lse_ref| <= 1e-3, over every compared row.

Every test compares every row it launches, element by element: the method is exact
and each row is independent, so no row may be skipped. The full-size workloads are
launched exactly as the benchmark launches them; the oracle then computes all their
rows on a thread pool of host cores (blocks of at most 256 rows, one BLAS thread per
worker), which takes from seconds (B=2, H=32, N=8192) to about a minute (H=16,
N=32768).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import ORACLE_WORKERS as WORKERS, one_blas_thread, parallel_map
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import WORKLOADS, make_inputs, random_tensor

pytestmark = pytest.mark.gpu

TOL_O = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    fa.load()
    yield
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)


def run_forward(q, k, v, scale, causal, poison=True):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, H, N, D = q.shape
    o = torch.empty(B, H, N, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    fa.fa_forward(qd, kd, vd, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, o_ref, lse_ref, dtype, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output (unwritten rows?)"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse - lse_ref))) if lse.size else 0.0
    say(f"{what}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
    assert err_o <= TOL_O[dtype], f"{what}: max|dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max|dlse| = {err_l}"


# ------------------------------------------------------------------ small and ragged sizes
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 1000])
def test_forward_sizes(dtype, D, causal, N):
    seed = 1000 * D + 10 * N + int(causal)
    q = random_tensor((2, 3, N, D), seed, dtype)
    k = random_tensor((2, 3, N, D), seed + 1, dtype)
    v = random_tensor((2, 3, N, D), seed + 2, dtype)
    scale = 1.0 / math.sqrt(D)
    say(f"forward N={N} D={D} causal={causal} dtype={dtype}")
    o, lse = run_forward(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    check(o, lse, o_ref, lse_ref, dtype, f"N={N} D={D} causal={causal}")


# ------------------------------------------------------------------ the named workloads
def test_single_head_fp32():
    w = WORKLOADS["single_head_fp32"]
    q, k, v = make_inputs(w)
    say(f"workload {w.name}")
    o, lse = run_forward(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    check(o, lse, o_ref, lse_ref, w.dtype, w.name)
    # The observed error should sit near the sqrt(N) u scale, far below the tolerance.
    assert float(np.max(np.abs(o - o_ref))) < 1e-5


@pytest.mark.parametrize("name", ["batched_prefill_d64", "batched_prefill_d64_causal"])
def test_batched_prefill_d64_full(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    say(f"workload {w.name} (all rows)")
    o, lse = run_forward(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal, workers=WORKERS)
    check(o, lse, o_ref, lse_ref, w.dtype, w.name)


def test_large_score_reduced_all_rows():
    """The large-score distribution (q, k ~ N(0, 9)) at a size compared in full."""
    w = WORKLOADS["large_score_causal_d128"]
    q, k, v = make_inputs(w, B=1, H=4, N=1031)
    say("large-score distribution, B=1 H=4 N=1031")
    o, lse = run_forward(q, k, v, w.scale, True)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, True, workers=WORKERS)
    check(o, lse, o_ref, lse_ref, w.dtype, "large-score N=1031")
    # raw scaled scores really reach the tens here
    s = w.scale * (q[0, 0, :64].double() @ k[0, 0].double().T)
    assert float(s.max()) > 30.0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["large_score_causal_d128", "long_context_causal_32768",
                                  "long_context_causal_32767"])
def test_full_size_prefill_all_rows(name):
    """The benchmark's launch at full size, every row of every head against the oracle."""
    w = WORKLOADS[name]
    say(f"workload {w.name}: drawing inputs")
    q, k, v = make_inputs(w)
    say(f"workload {w.name}: full-size launch")
    o, lse = run_forward(q, k, v, w.scale, w.causal, poison=True)
    say(f"workload {w.name}: oracle over all {w.B * w.H * w.N} rows, {WORKERS} workers")
    with one_blas_thread():
        o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal, row_block=256,
                                          workers=WORKERS)
    check(o, lse, o_ref, lse_ref, w.dtype, f"{w.name} (all rows)")


# ------------------------------------------------------------------ sizes past one tile row
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1031, 1537, 2049, 4095, 4097])
def test_forward_sizes_past_1024(D, causal, N):
    """Lengths just past and just short of whole 256-row query tiles and 64-key tiles,
    between 1024 and 2048 as well as past 2048, bf16, every row compared."""
    seed = 5000 + 3 * N + D + int(causal)
    q, k, v = (random_tensor((1, 2, N, D), seed + i, torch.bfloat16) for i in range(3))
    scale = 1.0 / math.sqrt(D)
    say(f"forward N={N} D={D} causal={causal}")
    o, lse = run_forward(q, k, v, scale, causal)
    with one_blas_thread():
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal, row_block=512,
                                          workers=WORKERS)
    check(o, lse, o_ref, lse_ref, torch.bfloat16, f"N={N} D={D} causal={causal}")


def _overflowing_fp32_inputs(shape_q, shape_kv, seed):
    """fp32 q, k ~ N(0, 4) at D = 64: with scale = 1 the raw scores reach well past
    ln(FLT_MAX) = 88.72, where e^s itself overflows float32."""
    q = random_tensor(shape_q, seed, torch.float32, sigma=2.0)
    k = random_tensor(shape_kv, seed + 1, torch.float32, sigma=2.0)
    v = random_tensor(shape_kv, seed + 2, torch.float32)
    return q, k, v


@pytest.mark.parametrize("scale", [1e-30, 400.0], ids=["tiny", "large"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_forward_extreme_scales(scale, D, causal):
    """The two ends of the softmax. A scale of 1e-30 makes every visible key weigh the
    same (O = mean of the visible values, lse = ln of their count). A scale of 400 puts
    the scaled scores near 2e4, where the largest score takes all the weight and every
    step whose block holds a new maximum goes through the rare path; that is about the
    largest magnitude the kernels' exponents (s c - m c in one fused multiply-add, c =
    scale log2 e) keep to bf16 precision, |m c| <= 2^15. lse is compared relative to its
    size there (float32 spacing at 2e4 is 2e-3)."""
    seed = 6100 + D + int(causal) + (7 if scale > 1 else 0)
    q, k, v = (random_tensor((1, 2, 300, D), seed + i, torch.bfloat16) for i in range(3))
    say(f"forward scale={scale:g} D={D} causal={causal}")
    o, lse = run_forward(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err_o = float(np.max(np.abs(o - o_ref)))
    err_l = float(np.max(np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))))
    say(f"max|dO|={err_o:.3e} max|dlse|/max(1,|lse|)={err_l:.3e} max|lse|={np.max(np.abs(lse_ref)):.3g}")
    assert err_o <= TOL_O[torch.bfloat16]
    assert err_l <= TOL_LSE * (1e-3 if scale > 1 else 1)


@pytest.mark.parametrize("scale", [1e-30, 400.0, 1e20], ids=["tiny", "large", "huge"])
def test_decode_extreme_scales(scale):
    """Split-KV decode at both ends of the softmax (see test_forward_extreme_scales). The
    decode subtracts each chunk's maximum before scaling, so it also holds at scaled
    scores near 1e21 (a scale of 1e20)."""
    q = random_tensor((1, 4, 1, 128), 6200, torch.bfloat16)
    k, v = (random_tensor((1, 4, 3000, 128), 6201 + i, torch.bfloat16) for i in range(2))
    _, _, _, o, lse = run_decode(q, k, v, scale, 16)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    err_o = float(np.max(np.abs(o - o_ref.reshape(4, 128))))
    lr = lse_ref.reshape(4)
    err_l = float(np.max(np.abs(lse - lr) / np.maximum(1.0, np.abs(lr))))
    say(f"decode scale={scale:g}: max|dO|={err_o:.3e} max|dlse|/max(1,|lse|)={err_l:.3e}")
    assert err_o <= TOL_O[torch.bfloat16]
    assert err_l <= TOL_LSE * (1e-3 if scale > 1 else 1)


def test_fp32_unscaled_scores_overflow_exp():
    """Safe softmax in float32: scale = 1 puts raw scores above 88.72, so e^s overflows
    float32 without the maximum subtracted ("Softmax Looks Like It Breaks the Rules");
    the fp32 kernel must still match the oracle to 1e-4 / 1e-3."""
    q, k, v = _overflowing_fp32_inputs((1, 2, 256, 64), (1, 2, 256, 64), 91)
    s = q[0, 0].double() @ k[0, 0].double().T
    assert float(s.max()) > 100.0
    assert torch.isinf(torch.exp(s.float())).any(), "e^s must overflow float32 here"
    for causal in (False, True):
        o, lse = run_forward(q, k, v, 1.0, causal)
        o_ref, lse_ref = oracle.attention(q, k, v, 1.0, causal)
        check(o, lse, o_ref, lse_ref, torch.float32, f"fp32 scale=1 causal={causal}")
        assert float(np.max(lse)) > 88.72


def test_fp32_decode_unscaled_scores_overflow_exp():
    """The same through the fp32 split-KV decode: partials and merge, scale = 1."""
    q, k, v = _overflowing_fp32_inputs((2, 2, 1, 64), (2, 2, 1000, 64), 93)
    s = torch.einsum("bhd,bhld->bhl", q[:, :, 0].double(), k.double())
    assert float(s.max()) > 88.72 and torch.isinf(torch.exp(s.float())).any()
    m, d, op, o, lse = run_decode(q, k, v, 1.0, 7)
    m_ref, d_ref, _ = oracle.decode_partials(q, k, v, 1.0, 7)
    assert np.max(np.abs(m - m_ref)) <= 1e-3 and float(np.max(m)) > 88.72
    f = np.exp(m - m_ref)
    assert np.max(np.abs(d * f - d_ref) / d_ref) <= 1e-3
    o_ref, lse_ref = oracle.attention(q, k, v, 1.0, False)
    check(o, lse, o_ref.reshape(4, 64), lse_ref.reshape(4), torch.float32, "fp32 decode scale=1")


# ------------------------------------------------------------------ closed forms through the kernels
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_come_back(dtype, causal):
    N, D = 300, 128
    q = random_tensor((1, 2, N, D), 1, dtype, sigma=3.0)
    k = random_tensor((1, 2, N, D), 2, dtype, sigma=3.0)
    vrow = random_tensor((D,), 3, dtype)
    v = vrow.expand(1, 2, N, D).contiguous()
    o, _ = run_forward(q, k, v, 1 / math.sqrt(D), causal)
    err = np.max(np.abs(o - vrow.double().numpy()))
    say(f"constant V: max err {err:.3e}")
    assert err <= TOL_O[dtype] / 4


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_and_log_count(causal):
    N, D = 257, 64
    q = random_tensor((1, 1, N, D), 4, torch.float32)
    krow = random_tensor((D,), 5, torch.float32)
    k = krow.expand(1, 1, N, D).contiguous()
    v = random_tensor((1, 1, N, D), 6, torch.float32)
    scale = 0.125
    o, lse = run_forward(q, k, v, scale, causal)
    vv = v[0, 0].double().numpy()
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vv, axis=0) / cnt[:, None] if causal else np.broadcast_to(vv.mean(0), vv.shape)
    s = scale * (q[0, 0].double().numpy() @ krow.double().numpy())
    assert np.max(np.abs(o[0, 0] - mean)) <= 1e-4
    assert np.max(np.abs(lse[0, 0] - (s + np.log(cnt)))) <= 1e-4


def test_single_key_and_row_zero():
    q = random_tensor((2, 2, 1, 128), 7)
    k = random_tensor((2, 2, 1, 128), 8)
    v = random_tensor((2, 2, 1, 128), 9)
    o, lse = run_forward(q, k, v, 0.1, False)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0].double().numpy(), atol=1e-6, rtol=0)
    s = 0.1 * (q.double() * k.double()).sum(-1).numpy()
    np.testing.assert_allclose(lse, s, atol=1e-4, rtol=0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_growing_scores_force_rescales(D, causal):
    """Scores that climb steeply along the keys: each 32-key block's maximum exceeds
    the previous one by about 2^40 in weight, so the running maximum moves on every
    block and the accumulator is rescaled every step (the reference-maximum change
    of coordinates, exercised on every step instead of rarely)."""
    N = 333
    q = random_tensor((1, 2, N, D), 21, torch.bfloat16)
    k = random_tensor((1, 2, N, D), 22, torch.bfloat16)
    v = random_tensor((1, 2, N, D), 23, torch.bfloat16)
    q[..., 0] = 1.0
    k[..., 0] = (10.0 * torch.arange(N, dtype=torch.float32)).to(torch.bfloat16)
    scale = 1 / math.sqrt(D)
    o, lse = run_forward(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    check(o, lse, o_ref, lse_ref, torch.bfloat16, f"growing scores D={D} causal={causal}")


def test_row_shift_invariance_fp32():
    N, D = 200, 64
    q = random_tensor((1, 1, N, D), 10, torch.float32)
    k = random_tensor((1, 1, N, D), 11, torch.float32)
    v = random_tensor((1, 1, N, D), 12, torch.float32)
    c = random_tensor((N,), 13, torch.float32) * 8
    q2, k2 = q.clone(), k.clone()
    q2[0, 0, :, -1] = c      # the last column carries c_i ...
    k2[0, 0, :, -1] = 2.0    # ... against a constant key column
    q2[0, 0, :, :-1] = q[0, 0, :, :-1]
    q1, k1 = q2.clone(), k2.clone()
    q1[0, 0, :, -1] = 0.0    # same scores without the per-row shift
    for causal in (False, True):
        o1, l1 = run_forward(q1, k1, v, 0.125, causal)
        o2, l2 = run_forward(q2, k2, v, 0.125, causal)
        assert np.max(np.abs(o2 - o1)) <= 1e-4
        assert np.max(np.abs(l2[0, 0] - l1[0, 0] - 0.125 * 2.0 * c.double().numpy())) <= 1e-3


def test_key_permutation_noncausal():
    N, D = 700, 128
    q, k, v = (random_tensor((1, 2, N, D), 20 + i) for i in range(3))
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(3))
    o1, l1 = run_forward(q, k, v, 1 / math.sqrt(D), False)
    o2, l2 = run_forward(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 1 / math.sqrt(D), False)
    assert np.max(np.abs(o1 - o2)) <= 2e-2 and np.max(np.abs(l1 - l2)) <= 1e-3


def test_deterministic_and_stream_ordered():
    w = WORKLOADS["batched_prefill_d64_causal"]
    q, k, v = (t.cuda() for t in make_inputs(w, B=1, H=4, N=777))
    outs = []
    s = torch.cuda.Stream()
    for stream in (None, s):
        o = torch.full((1, 4, 777, 64), float("nan"), device="cuda")
        lse = torch.full((1, 4, 777), float("nan"), device="cuda")
        with torch.cuda.stream(s if stream is not None else torch.cuda.current_stream()):
            fa.fa_forward(q, k, v, o, lse, w.scale, True, stream)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_empty_problems_touch_nothing():
    z = torch.zeros(1, 1, 0, 64, dtype=torch.bfloat16, device="cuda")
    oz = torch.zeros(1, 1, 0, 64, device="cuda")
    lz = torch.zeros(1, 1, 0, device="cuda")
    fa.fa_forward(z, z, z, oz, lz, 0.125, False)  # N = 0: NULL data pointers are fine
    guard = torch.full((64,), 7.0, device="cuda")
    fa.fa_combine_partials(torch.zeros(0, 3, device="cuda"), torch.zeros(0, 3, device="cuda"),
                           torch.zeros(0, 3, 64, device="cuda"), torch.zeros(0, 64, device="cuda"),
                           torch.zeros(0, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(guard == 7.0)


def test_decode_with_no_keys_writes_identities():
    q = random_tensor((1, 2, 1, 128), 40)
    k = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16)
    m, d, op, o, lse = run_decode(q, k, k, 0.1, 4)
    assert np.all(np.isneginf(m)) and np.all(d == 0) and np.all(op == 0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------------------------ split-KV decode
def run_decode(q, k, v, scale, splits):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, H, L, D = k.shape
    m = torch.full((B * H, splits), float("nan"), device="cuda")
    d = torch.full((B * H, splits), float("nan"), device="cuda")
    op = torch.full((B * H, splits, D), float("nan"), device="cuda")
    o = torch.full((B * H, D), float("nan"), device="cuda")
    lse = torch.full((B * H,), float("nan"), device="cuda")
    fa.fa_decode_partials(qd, kd, vd, m, d, op, scale, splits)
    fa.fa_combine_partials(m, d, op, o, lse)
    torch.cuda.synchronize()
    return [t.cpu().double().numpy() for t in (m, d, op, o, lse)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("L,splits", [(1, 1), (100, 1), (100, 7), (513, 4), (1000, 64), (4096, 8), (5, 8)])
def test_decode_sizes(dtype, D, L, splits):
    seed = 7 * L + splits + D
    q = random_tensor((2, 3, 1, D), seed, dtype)
    k = random_tensor((2, 3, L, D), seed + 1, dtype, sigma=2.0)
    v = random_tensor((2, 3, L, D), seed + 2, dtype)
    scale = 1 / math.sqrt(D)
    say(f"decode L={L} splits={splits} D={D} dtype={dtype}")
    m, d, op, o, lse = run_decode(q, k, v, scale, splits)
    m_ref, d_ref, op_ref = oracle.decode_partials(q, k, v, scale, splits)
    empty = np.isneginf(m_ref)
    assert np.array_equal(np.isneginf(m), empty)
    assert np.all(d[empty] == 0) and np.all(op[empty] == 0)
    ne = ~empty
    assert np.max(np.abs(m[ne] - m_ref[ne])) <= 1e-3
    # d, o are relative to m: compare after bringing both to the oracle's reference
    f = np.exp(m[ne] - m_ref[ne])
    assert np.max(np.abs(d[ne] * f - d_ref[ne]) / d_ref[ne]) <= 1e-3
    chunk = -(-L // splits)
    assert np.all(d[ne] >= 1 - 1e-5) and np.all(d[ne] <= chunk + 1e-3)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    check(o, lse, o_ref.reshape(6, D), lse_ref.reshape(6), dtype, f"decode L={L} splits={splits}")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16", "fp32"])
@pytest.mark.parametrize("B,H,L,splits", [(1, 1, 200, 1), (1, 3, 300, 5), (1, 1, 513, 3),
                                          (3, 1, 1000, 7)])
def test_decode_odd_unit_counts(dtype, D, B, H, L, splits):
    """B * H * splits odd: a workgroup folds two (head, chunk) units in turn, so the last
    workgroup has a single unit and must stop after it."""
    seed = 11 * L + splits + B
    q = random_tensor((B, H, 1, D), seed, dtype)
    k = random_tensor((B, H, L, D), seed + 1, dtype, sigma=2.0)
    v = random_tensor((B, H, L, D), seed + 2, dtype)
    scale = 1 / math.sqrt(D)
    say(f"decode odd units B={B} H={H} L={L} splits={splits} D={D} dtype={dtype}")
    m, d, op, o, lse = run_decode(q, k, v, scale, splits)
    m_ref, d_ref, op_ref = oracle.decode_partials(q, k, v, scale, splits)
    assert np.array_equal(np.isneginf(m), np.isneginf(m_ref))
    ne = ~np.isneginf(m_ref)
    assert np.max(np.abs(m[ne] - m_ref[ne])) <= 1e-3
    f = np.exp(m[ne] - m_ref[ne])
    assert np.max(np.abs(d[ne] * f - d_ref[ne]) / d_ref[ne]) <= 1e-3
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    check(o, lse, o_ref.reshape(B * H, D), lse_ref.reshape(B * H), dtype,
          f"decode odd units B={B} H={H} L={L} splits={splits}")


def _decode_head_reference(q, k, v, scale, splits, b, h):
    """The oracle for one head: its partial states, their fold, and the plain definition."""
    sl = (slice(b, b + 1), slice(h, h + 1))
    m_ref, d_ref, op_ref = oracle.decode_partials(q[sl], k[sl], v[sl], scale, splits)
    o_ref, lse_ref = oracle.attention(q[sl], k[sl], v[sl], scale, False)
    return m_ref[0], d_ref[0], op_ref[0], o_ref.reshape(-1), float(lse_ref.reshape(-1)[0])


def _check_decode_heads(q, k, v, scale, splits, m, d, op, o, lse, what):
    """Every head: partials (m exactly in natural-log units; d and o after rebasing to the
    oracle's m), the merged output and lse."""
    B, H = k.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)]
    with one_blas_thread():
        refs = parallel_map(lambda bh: _decode_head_reference(q, k, v, scale, splits, *bh), heads)
    m_ref = np.stack([r[0] for r in refs])
    d_ref = np.stack([r[1] for r in refs])
    op_ref = np.stack([r[2] for r in refs])
    o_ref = np.stack([r[3] for r in refs])
    lse_ref = np.array([r[4] for r in refs])
    empty = np.isneginf(m_ref)
    assert np.array_equal(np.isneginf(m), empty), f"{what}: identity partials"
    ne = ~empty
    assert np.max(np.abs(m[ne] - m_ref[ne])) <= 1e-3, f"{what}: partial maxima"
    f = np.exp(m - np.where(empty, 0.0, m_ref))
    f[empty] = 0.0
    assert np.max(np.abs(d[ne] * f[ne] - d_ref[ne]) / d_ref[ne]) <= 1e-3, f"{what}: partial d"
    err_op = np.abs(op * f[..., None] - op_ref).max(axis=-1) / np.maximum(d_ref, 1.0)
    assert float(err_op.max()) <= 2e-2, f"{what}: partial o (relative to d) {err_op.max()}"
    check(o, lse, o_ref, lse_ref, torch.bfloat16, f"{what} ({len(heads)} heads)")
    return o_ref, lse_ref


@pytest.mark.timeout(900)
def test_split_kv_decode_full_size():
    """The benchmark's decode at full size (B=16, H=32, L=32768, 64 chunks): every
    partial of every head and every merged row against the oracle. Then the same keys
    cut into 8 shards of 4096 (one GPU's share of an 8-GPU split), each shard's 64
    partials produced by its own fa_decode_partials call, and all 8 x 64 remote-shaped
    partials merged by one fa_combine_partials call."""
    w = WORKLOADS["split_kv_decode"]
    say(f"workload {w.name}: drawing inputs")
    q, k, v = make_inputs(w)
    say("running decode at full size")
    m, d, op, o, lse = run_decode(q, k, v, w.scale, w.splits)
    chunk = w.L // w.splits
    assert np.all(d >= 1 - 1e-5) and np.all(d <= chunk + 1e-3), "1 <= d <= chunk length"
    say("oracle over all 512 heads")
    o_ref, lse_ref = _check_decode_heads(q, k, v, w.scale, w.splits, m, d, op, o, lse, w.name)

    shards, per = 8, w.L // 8
    say(f"{shards} shards of {per} keys, {w.splits} partials each, merged at once")
    qd = q.cuda()
    BH = w.B * w.H
    ms = torch.empty(BH, shards, w.splits, device="cuda")
    ds = torch.empty(BH, shards, w.splits, device="cuda")
    ops = torch.empty(BH, shards, w.splits, w.D, device="cuda")
    for s in range(shards):
        ks = k[:, :, s * per:(s + 1) * per].contiguous().cuda()
        vs = v[:, :, s * per:(s + 1) * per].contiguous().cuda()
        mp, dp = torch.empty(BH, w.splits, device="cuda"), torch.empty(BH, w.splits, device="cuda")
        opp = torch.empty(BH, w.splits, w.D, device="cuda")
        fa.fa_decode_partials(qd, ks, vs, mp, dp, opp, w.scale, w.splits)
        ms[:, s], ds[:, s], ops[:, s] = mp, dp, opp
        del ks, vs
    o2 = torch.full((BH, w.D), float("nan"), device="cuda")
    l2 = torch.full((BH,), float("nan"), device="cuda")
    fa.fa_combine_partials(ms.view(BH, -1), ds.view(BH, -1), ops.view(BH, -1, w.D), o2, l2)
    torch.cuda.synchronize()
    check(o2.cpu().double().numpy(), l2.cpu().double().numpy(), o_ref, lse_ref, w.dtype,
          f"{w.name}, {shards} shards x {w.splits} partials")


@pytest.mark.parametrize("splits", [8, 64])
def test_split_kv_decode_one_gpu_share(splits):
    """One GPU's share of the decode workload split over 8 GPUs: B=16, H=32, L=4096 keys
    per head, in 8 or 64 chunks; every partial and every merged row compared."""
    w = WORKLOADS["split_kv_decode"]
    q, k, v = make_inputs(w, L=4096)
    say(f"decode share L=4096 splits={splits}")
    m, d, op, o, lse = run_decode(q, k, v, w.scale, splits)
    _check_decode_heads(q, k, v, w.scale, splits, m, d, op, o, lse, f"share splits={splits}")


def test_combine_split_count_and_order_invariance():
    L, D = 4096, 128
    q = random_tensor((1, 4, 1, D), 30)
    k = random_tensor((1, 4, L, D), 31, sigma=2.0)
    v = random_tensor((1, 4, L, D), 32)
    scale = 1 / math.sqrt(D)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    for splits in (1, 2, 8, 64):
        m, d, op, o, lse = run_decode(q, k, v, scale, splits)
        check(o, lse, o_ref.reshape(4, D), lse_ref.reshape(4), torch.bfloat16, f"splits={splits}")
        perm = np.random.default_rng(splits).permutation(splits)
        mt, dt, opt = (torch.tensor(x[:, perm], dtype=torch.float32).contiguous().cuda()
                       for x in (m, d, op))
        o2 = torch.empty(4, D, device="cuda")
        l2 = torch.empty(4, device="cuda")
        fa.fa_combine_partials(mt, dt, opt, o2, l2)
        torch.cuda.synchronize()
        assert np.max(np.abs(o2.cpu().double().numpy() - o)) <= 1e-5
        assert np.max(np.abs(l2.cpu().double().numpy() - lse)) <= 1e-5


def test_combine_all_identity_rows():
    m = torch.full((3, 5), float("-inf"), device="cuda")
    d = torch.zeros(3, 5, device="cuda")
    op = torch.zeros(3, 5, 64, device="cuda")
    m[1, 2], d[1, 2], op[1, 2] = 0.5, 2.0, 4.0
    o = torch.full((3, 64), float("nan"), device="cuda")
    lse = torch.full((3,), float("nan"), device="cuda")
    fa.fa_combine_partials(m, d, op, o, lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.all(o[0] == 0) and torch.all(o[2] == 0)
    assert math.isinf(lse[0]) and lse[0] < 0 and math.isinf(lse[2])
    assert torch.allclose(o[1], torch.full((64,), 2.0)) and abs(lse[1] - (0.5 + math.log(2.0))) < 1e-6


def test_repeated_launches_write_every_row_identically():
    """600 launches alternating two causal shapes (more query tiles than CUs, tiles of
    different lengths): every launch writes every row (outputs start as NaN) and equals
    the first launch of its shape bit for bit. The library keeps no state between
    calls, so nothing may leak from one launch into the next."""
    shapes = [(4, 16, 4096, 64), (2, 16, 1536, 128)]
    runs = []
    for i, (B, H, N, D) in enumerate(shapes):
        q, k, v = (random_tensor((B, H, N, D), 4000 + 10 * i + j).cuda() for j in range(3))
        o = torch.empty(B, H, N, D, device="cuda")
        lse = torch.empty(B, H, N, device="cuda")
        runs.append((q, k, v, o, lse, 1 / math.sqrt(D)))
    first = [None, None]
    for n in range(600):
        q, k, v, o, lse, scale = runs[n % 2]
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        fa.fa_forward(q, k, v, o, lse, scale, True)
        if first[n % 2] is None:
            first[n % 2] = (o.clone(), lse.clone())
            assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        else:
            assert torch.equal(o, first[n % 2][0]), f"launch {n}: output differs"
            assert torch.equal(lse, first[n % 2][1]), f"launch {n}: lse differs"
    torch.cuda.synchronize()
    say("600 launches: every row written, identical outputs")
