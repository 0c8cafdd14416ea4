"""Seeded random sweep: shapes, scales, masks and split counts drawn at random (from a
fixed seed, so every run draws the same cases), each call compared with the fp64
oracle on every row it writes. The hand-picked sizes of the other tests sit on tile
edges; these land anywhere, in combinations nobody chose.

Tolerances are those of the other parity tests: O within 2e-2 (bfloat16 inputs) or 1e-4
(float32 inputs) absolute, lse within 1e-3; gradients within 1e-2 (bfloat16) or 1e-4
(float32) of max(1, max |g_ref|); decode partials' maxima within 1e-3 and their
denominators within 1e-3 relative after rebasing to the oracle's maxima, their o within
2e-2 (bfloat16) or 1e-3 (float32) of max(1, d_ref). Outputs start
as NaN, so a row a kernel misses fails, and rows a call must not write must stay NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import random_tensor

pytestmark = pytest.mark.gpu

TOL_O = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
TOL_LSE = 1e-3
TOL_GRAD = {torch.bfloat16: 1e-2, torch.float32: 1e-4}
TOL_PART_O = {torch.bfloat16: 2e-2, torch.float32: 1e-3}  # relative to max(1, d_ref)
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    fa.load()
    yield
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)


def _window(rng, n):
    """A random window side: unbounded, zero, small, or past the sequence."""
    r = rng.random()
    if r < 0.25:
        return -1
    if r < 0.35:
        return 0
    if r < 0.85:
        return int(rng.integers(1, max(2, n)))
    return int(rng.integers(n, n + 2000))


def _dense_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        D = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 2200))
        bh = max(1, min(6, int(4e6 // max(N * N, 1))))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, max(2, bh // B + 1)))
        cases.append(dict(i=i, B=B, H=H, N=N, D=D, causal=bool(rng.integers(0, 2)),
                          scale=float(rng.uniform(0.3, 2.0) / math.sqrt(D)),
                          sigma=float(rng.choice([1.0, 1.0, 3.0])),
                          wl=_window(rng, N), wr=_window(rng, N), seed=int(rng.integers(1, 2**30))))
    return cases


def _name(c):
    return f"B{c['B']}H{c['H']}N{c['N']}D{c['D']}{'c' if c['causal'] else 'f'}"


DENSE = _dense_cases(24, 20261203)
WINDOWED = _dense_cases(24, 20261204)


def _inputs(c, dtype, n_tensors=3, sigma_qk=None):
    sig = c["sigma"] if sigma_qk is None else sigma_qk
    shape = (c["B"], c["H"], c["N"], c["D"])
    return [random_tensor(shape, c["seed"] + i, dtype, sigma=sig if i < 2 else 1.0)
            for i in range(n_tensors)]


def _check_o(o, lse, o_ref, lse_ref, dtype, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output (unwritten rows?)"
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: -inf pattern"
    fin = np.isfinite(lse_ref)
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    say(f"{what}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
    assert err_o <= TOL_O[dtype], f"{what}: max|dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max|dlse| = {err_l}"


def _nan_outputs(shape):
    o = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("c", DENSE, ids=_name)
def test_random_forward(c, dt):
    dtype = DT[dt]
    sigma = c["sigma"] if dtype == torch.bfloat16 else 1.0
    q, k, v = _inputs(c, dtype, sigma_qk=sigma)
    what = f"forward {dt} {c}"
    say(what)
    o, lse = _nan_outputs(tuple(q.shape))
    fa.fa_forward(q.cuda(), k.cuda(), v.cuda(), o, lse, c["scale"], c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, c["scale"], c["causal"])
    _check_o(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, dtype, what)


@pytest.mark.parametrize("c", WINDOWED, ids=_name)
def test_random_window(c):
    q, k, v = _inputs(c, torch.bfloat16)
    what = f"window {c}"
    say(what)
    o, lse = _nan_outputs(tuple(q.shape))
    fa.fa_forward_ext(q.cuda(), k.cuda(), v.cuda(), o, lse, c["scale"], c["causal"], c["wl"],
                      c["wr"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_window(q, k, v, c["scale"], c["causal"], c["wl"], c["wr"])
    _check_o(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
             torch.bfloat16, what)


def _varlen_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        nseq = int(rng.integers(1, 11))
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 900, nseq)]
        longest = max(lens + [1])
        cases.append(dict(i=i, lens=lens, H=int(rng.integers(1, 4)), D=int(rng.choice([64, 128])),
                          causal=bool(rng.integers(0, 2)), wl=_window(rng, longest),
                          wr=_window(rng, longest), extra=int(rng.integers(0, 70)),
                          scale=float(rng.uniform(0.3, 2.0)), seed=int(rng.integers(1, 2**30))))
    return cases


VARLEN = _varlen_cases(12, 20261205)


@pytest.mark.parametrize("c", VARLEN, ids=lambda c: f"nseq{len(c['lens'])}D{c['D']}")
def test_random_varlen(c):
    D = c["D"]
    cu = np.concatenate([[0], np.cumsum(c["lens"])]).astype(np.int32)
    total = int(cu[-1]) + c["extra"]  # rows past the last sequence: no call may write them
    scale = c["scale"] / math.sqrt(D)
    q, k, v = (random_tensor((c["H"], total, D), c["seed"] + i, torch.bfloat16) for i in range(3))
    what = f"varlen {c}"
    say(what)
    o, lse = _nan_outputs((c["H"], total, D))
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    fa.fa_forward_ext(q.cuda(), k.cuda(), v.cuda(), o, lse, scale, c["causal"], c["wl"], c["wr"],
                      cud, max(c["lens"]))
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    n = int(cu[-1])
    o_ref, lse_ref = oracle.attention_varlen(q[:, :n], k[:, :n], v[:, :n], cu, scale, c["causal"],
                                             c["wl"], c["wr"])
    _check_o(o[:, :n], lse[:, :n], o_ref, lse_ref, torch.bfloat16, what)
    assert np.all(np.isnan(o[:, n:])) and np.all(np.isnan(lse[:, n:])), "rows past cu[-1] written"


def _backward_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        D = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 1300))
        cases.append(dict(i=i, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), N=N, D=D,
                          causal=bool(rng.integers(0, 2)),
                          scale=float(rng.uniform(0.3, 2.0) / math.sqrt(D)),
                          sigma=float(rng.choice([1.0, 2.0])), seed=int(rng.integers(1, 2**30)),
                          dt=str(rng.choice(["bf16", "bf16", "fp32"]))))
    return cases


BACKWARD = _backward_cases(16, 20261206)


@pytest.mark.parametrize("c", BACKWARD, ids=lambda c: _name(c) + c["dt"])
def test_random_backward(c):
    dtype = DT[c["dt"]]
    q, k, v, do = _inputs(c, dtype, n_tensors=4)
    what = f"backward {c}"
    say(what)
    qd, kd, vd, dd = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, c["scale"], c["causal"])
    shape = tuple(q.shape)
    delta = torch.empty(shape[:-1], dtype=torch.float32, device="cuda")
    grads = [torch.full(shape, float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    fa.fa_backward(qd, kd, vd, o, lse, dd, delta, *grads, c["scale"], c["causal"])
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, do, c["scale"], c["causal"])[:3]
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        g = g.cpu().double().numpy()
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite output"
        err = float(np.max(np.abs(g - r)))
        lim = TOL_GRAD[dtype] * max(1.0, float(np.max(np.abs(r))))
        say(f"{name}: max|err| {err:.3e} (limit {lim:.3e})")
        assert err <= lim, f"{what} {name}: {err} > {lim}"


def _decode_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        D = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 7000))
        cases.append(dict(i=i, B=int(rng.integers(1, 4)), H=int(rng.integers(1, 5)), L=L, D=D,
                          splits=int(rng.integers(1, 130)),
                          scale=float(rng.uniform(0.3, 2.0) / math.sqrt(D)),
                          sigma=float(rng.choice([1.0, 2.0, 3.0])), seed=int(rng.integers(1, 2**30)),
                          dt=str(rng.choice(["bf16", "bf16", "fp32"]))))
    return cases


DECODE = _decode_cases(16, 20261207)


@pytest.mark.parametrize("c", DECODE, ids=lambda c: f"B{c['B']}H{c['H']}L{c['L']}s{c['splits']}{c['dt']}")
def test_random_decode(c):
    dtype = DT[c["dt"]]
    B, H, L, D, splits = c["B"], c["H"], c["L"], c["D"], c["splits"]
    q = random_tensor((B, H, 1, D), c["seed"], dtype)
    k = random_tensor((B, H, L, D), c["seed"] + 1, dtype, sigma=c["sigma"])
    v = random_tensor((B, H, L, D), c["seed"] + 2, dtype)
    what = f"decode {c}"
    say(what)
    rows = B * H
    m = torch.full((rows, splits), float("nan"), device="cuda")
    d = torch.full((rows, splits), float("nan"), device="cuda")
    op = torch.full((rows, splits, D), float("nan"), device="cuda")
    o = torch.full((rows, D), float("nan"), device="cuda")
    lse = torch.full((rows,), float("nan"), device="cuda")
    fa.fa_decode_partials(q.cuda(), k.cuda(), v.cuda(), m, d, op, c["scale"], splits)
    fa.fa_combine_partials(m, d, op, o, lse)
    torch.cuda.synchronize()
    m, d, op, o, lse = (t.cpu().double().numpy() for t in (m, d, op, o, lse))
    m_ref, d_ref, op_ref = oracle.decode_partials(q, k, v, c["scale"], splits)
    empty = np.isneginf(m_ref)
    assert np.array_equal(np.isneginf(m), empty), f"{what}: identity partials"
    assert np.all(d[empty] == 0) and np.all(op[empty] == 0), f"{what}: empty chunks"
    ne = ~empty
    assert np.max(np.abs(m[ne] - m_ref[ne])) <= 1e-3, f"{what}: partial maxima"
    f = np.exp(m[ne] - m_ref[ne])
    assert np.max(np.abs(d[ne] * f - d_ref[ne]) / d_ref[ne]) <= 1e-3, f"{what}: partial d"
    err_op = np.abs(op[ne] * f[:, None] - op_ref[ne]).max(axis=-1) / np.maximum(d_ref[ne], 1.0)
    assert float(err_op.max()) <= TOL_PART_O[dtype], f"{what}: partial o {err_op.max()}"
    o_ref, lse_ref = oracle.attention(q, k, v, c["scale"], False)
    _check_o(o, lse, o_ref.reshape(rows, D), lse_ref.reshape(rows), dtype, what)


# ------------------------------------------------------------------ row reductions and scans
# Random row counts, lengths, element offsets (rows on and off 16-byte boundaries),
# dtypes and value ranges, some scores at -inf; the bounds are those of the reduction
# and scan tests (tests/test_gpu_reductions.py, tests/test_gpu_scans.py), whose helpers
# run and check the calls.
from tests import test_gpu_reductions as _red  # noqa: E402
from tests import test_gpu_scans as _scan  # noqa: E402


def _row_cases(count, seed, max_n):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        cases.append(dict(i=i, rows=int(rng.integers(1, 41)), n=int(rng.integers(1, max_n)),
                          dt=str(rng.choice(["bf16", "fp32"])), offset=int(rng.integers(0, 8)),
                          sigma=float(rng.choice([0.5, 4.0, 30.0])),
                          mean=float(rng.choice([0.0, 3.0, -100.0])),
                          masked=float(rng.choice([0.0, 0.0, 0.3])),
                          seed=int(rng.integers(1, 2**30))))
    return cases


def _row_input(c, masked_ok):
    x = random_tensor((c["rows"], c["n"]), c["seed"], torch.float32, sigma=c["sigma"]) + c["mean"]
    if masked_ok and c["masked"] > 0:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(c["seed"] + 1)
        x[torch.rand(x.shape, generator=gen) < c["masked"]] = float("-inf")
    return x.to(DT[c["dt"]])


REDUCE = _row_cases(16, 20261208, 40000)
SCAN = _row_cases(16, 20261209, 9000)


@pytest.mark.parametrize("c", REDUCE, ids=lambda c: f"r{c['rows']}n{c['n']}{c['dt']}o{c['offset']}")
def test_random_row_reductions(c):
    what = f"reductions {c}"
    say(what)
    x = _row_input(c, True)
    m, d = _red.run(fa.fa_softmax_stats, x, c["offset"])
    _red.check_softmax(x, m, d, "softmax_stats " + what)
    x = _row_input(c, False)
    mean, m2 = _red.run(fa.fa_moments, x, c["offset"])
    _red.check_moments(x, mean, m2, "moments " + what)


@pytest.mark.parametrize("c", SCAN, ids=lambda c: f"r{c['rows']}n{c['n']}{c['dt']}o{c['offset']}")
def test_random_row_scans(c):
    what = f"scans {c}"
    say(what)
    x = _row_input(c, True)
    m, d = _scan.run(fa.fa_softmax_scan, x, c["offset"])
    _scan.check_softmax_scan(x, m, d, "softmax_scan " + what)
    x = _row_input(c, False)
    mean, m2 = _scan.run(fa.fa_moments_scan, x, c["offset"])
    _scan.check_moments_scan(x, mean, m2, "moments_scan " + what)
