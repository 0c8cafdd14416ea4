"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on one MI355X.

Tolerances: max |O - O_ref| <= 2e-2 absolute for bfloat16 inputs and <= 1e-4 for
float32 inputs, max |lse - lse_ref| <= 1e-3, over every compared row.

Sizes the oracle finishes in seconds are compared element by element over all rows;
the full-size workloads are launched exactly as the benchmark launches them and
compared on sampled rows, which the oracle computes one at a time.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import WORKLOADS, make_inputs, random_tensor

pytestmark = pytest.mark.gpu

TOL_O = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
TOL_LSE = 1e-3
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


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


def _sample_rows(B, H, N, per_head, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    rows = []
    for b in range(B):
        for h in range(H):
            picks = set(i for i in fixed if 0 <= i < N)
            picks.update(int(x) for x in rng.integers(0, N, per_head))
            rows += [(b, h, i) for i in sorted(picks)]
    return rows


@pytest.mark.parametrize("name", ["large_score_causal_d128", "long_context_causal_32768",
                                  "long_context_causal_32767"])
def test_full_size_prefill_sampled_rows(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    say(f"workload {w.name} full size, sampled rows")
    o, lse = run_forward(q, k, v, w.scale, w.causal, poison=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "unwritten or non-finite rows"
    rows = _sample_rows(w.B, w.H, w.N, 3 if w.B * w.H >= 32 else 8, seed=w.seed)
    o_ref, lse_ref = oracle.attention_selected_rows(q, k, v, w.scale, w.causal, rows)
    idx = tuple(np.array(rows).T)
    check(o[idx], lse[idx], o_ref, lse_ref, w.dtype, f"{w.name} ({len(rows)} rows)")


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


def test_split_kv_decode_full_size():
    w = WORKLOADS["split_kv_decode"]
    say(f"workload {w.name}: drawing inputs")
    q, k, v = make_inputs(w)
    say("running decode at full size")
    m, d, op, o, lse = run_decode(q, k, v, w.scale, w.splits)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    chunk = w.L // w.splits
    assert np.all(d >= 1 - 1e-5) and np.all(d <= chunk + 1e-3), "1 <= d <= chunk length"
    heads = [(0, 0), (0, 31), (7, 13), (15, 31), (9, 2), (3, 30)]
    for b, h in heads:
        r = b * w.H + h
        m_ref, d_ref, op_ref = oracle.decode_partials(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                                      v[b:b + 1, h:h + 1], w.scale, w.splits)
        assert np.max(np.abs(m[r] - m_ref[0])) <= 1e-3
        f = np.exp(m[r] - m_ref[0])
        assert np.max(np.abs(op[r] * f[:, None] - op_ref[0])) <= 2e-2 * np.max(d_ref[0])
        o_ref, lse_ref = oracle.combine_partials(m_ref, d_ref, op_ref)
        check(o[r:r + 1], lse[r:r + 1], o_ref, lse_ref, w.dtype, f"{w.name} head ({b},{h})")


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
