"""Parity of the row reductions (fa_softmax_stats, fa_moments, through the C ABI) with
the fp64 oracle, on one MI355X.

Tolerances, derived from the kernels' float32 arithmetic (unit roundoff u = 2^-24):
* m (softmax): exact. It is the maximum of the inputs, which float32 holds exactly.
* d (softmax): relative (n/64 + 32) * 2u. A lane adds at most n/64 block sums in
  sequence, each block 8 terms, then 6 butterfly and 3 wavefront merges; every
  rescale and every term passes through one hardware exp2 (<= 1 ulp) of an argument
  (x - m) log2(e) rounded twice, whose error only matters for terms near e^0.
* mean (moments): absolute (n/64 + 32) * 2u * max|x|: a lane's running mean moves
  by rounded steps at most n/64 + 8 times, and the merges add a few more.
* M2 (moments): relative (n/64 + 32) * 4u * max|x| / sigma, sigma^2 = M2 / n: the
  mean's error enters M2 through the merges' delta^2 term, at most twice its size
  times sqrt(n M2), on top of the block sums' own rounding (the usual conditioning
  of a variance, which is why a large common offset loosens it).
Inputs start at element offsets 0 and odd ones (a slice of a larger buffer), so rows
begin off 16-byte boundaries and the head, body and tail paths all run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import parallel_map
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import ROW_WORKLOADS, make_rows, random_tensor

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    fa.load()
    yield
    torch.cuda.synchronize()


def say(msg):
    print(msg, flush=True)


def on_gpu(x, offset=0):
    """x on the device, starting `offset` elements into a larger buffer."""
    rows, n = x.shape
    buf = torch.empty(rows * n + offset + 8, dtype=x.dtype, device="cuda")
    buf.fill_(float("nan"))
    view = buf[offset:offset + rows * n].view(rows, n)
    view.copy_(x.cuda())
    return view


def run(fn, x, offset=0):
    xd = on_gpu(x, offset)
    a, b = (torch.full((x.shape[0],), float("nan"), device="cuda") for _ in range(2))
    fn(xd, a, b)
    torch.cuda.synchronize()
    return a.cpu().double().numpy(), b.cpu().double().numpy()


def check_softmax(x, m, d, what):
    m_ref, d_ref = oracle.softmax_stats(x)
    n = x.shape[1]
    assert np.array_equal(m, m_ref), f"{what}: m not the exact maximum"
    live = d_ref > 0
    assert np.all(d[~live] == 0), f"{what}: identity rows"
    err = float(np.max(np.abs(d[live] - d_ref[live]) / d_ref[live])) if live.any() else 0.0
    tol = (n / 64 + 32) * 2 * U
    say(f"{what}: max rel err d {err:.3e} (tol {tol:.3e})")
    assert err <= tol, f"{what}: {err} > {tol}"


def check_moments(x, mean, m2, what):
    _, mu_ref, m2_ref = oracle.moments(x)
    n = x.shape[1]
    if n == 0:
        assert np.all(mean == 0) and np.all(m2 == 0)
        return
    xa = np.abs(x.double().numpy()).max(axis=1)
    tol_mu = (n / 64 + 32) * 2 * U * np.maximum(xa, 1e-30)
    err_mu = np.abs(mean - mu_ref)
    assert np.all(err_mu <= tol_mu), f"{what}: mean {np.max(err_mu / tol_mu)} x tol"
    sigma = np.sqrt(m2_ref / n)
    pos = m2_ref > 0
    tol_m2 = (n / 64 + 32) * 4 * U * (xa[pos] / sigma[pos])
    rel = np.abs(m2[pos] - m2_ref[pos]) / m2_ref[pos]
    assert np.all(m2[~pos] <= 4 * U * xa[~pos] ** 2 * n), f"{what}: constant rows"
    say(f"{what}: max |dmean| {np.max(err_mu):.3e}, max rel err M2 {np.max(rel, initial=0):.3e}")
    assert np.all(rel <= tol_m2), f"{what}: M2 {np.max(rel / tol_m2)} x tol"


DTYPES = [torch.float32, torch.bfloat16]
SIZES = [0, 1, 5, 7, 8, 9, 63, 64, 65, 1000, 4097, 33000]


@pytest.mark.parametrize("dtype", DTYPES, ids=["fp32", "bf16"])
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 3])
def test_softmax_stats_sizes(dtype, n, offset):
    rows = 37
    x = random_tensor((rows, n), 10 * n + offset, dtype, sigma=6.0)
    say(f"softmax_stats n={n} dtype={dtype} offset={offset}")
    m, d = run(fa.fa_softmax_stats, x, offset)
    check_softmax(x, m, d, f"softmax n={n} {dtype} off={offset}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["fp32", "bf16"])
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 5])
def test_moments_sizes(dtype, n, offset):
    rows = 37
    x = random_tensor((rows, n), 20 * n + offset, dtype, sigma=2.0)
    say(f"moments n={n} dtype={dtype} offset={offset}")
    mean, m2 = run(fa.fa_moments, x, offset)
    check_moments(x, mean, m2, f"moments n={n} {dtype} off={offset}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["fp32", "bf16"])
def test_many_rows_one_wavefront_each(dtype):
    """Enough rows for the one-wavefront-per-row schedule, with a ragged row count."""
    x = random_tensor((9001, 300), 31, dtype, sigma=5.0)
    m, d = run(fa.fa_softmax_stats, x, 1)
    check_softmax(x, m, d, f"softmax 9001 rows {dtype}")
    mean, m2 = run(fa.fa_moments, x, 1)
    check_moments(x, mean, m2, f"moments 9001 rows {dtype}")


def test_softmax_masked_and_extreme_scores():
    """-inf entries are the identity; all -inf rows give (-inf, 0); scores of +-3000
    would overflow any unshifted exponential."""
    x = random_tensor((50, 2000), 41, torch.float32, sigma=1000.0)
    x[x < -500] = -math.inf
    x[7] = -math.inf
    x[8, :1999] = -math.inf  # one live element: d = 1
    m, d = run(fa.fa_softmax_stats, x, 2)
    assert m[7] == -math.inf and d[7] == 0 and d[8] == 1.0
    check_softmax(x, m, d, "masked/extreme")


def test_softmax_constant_rows_count():
    x = torch.full((6, 777), 2.5)
    m, d = run(fa.fa_softmax_stats, x)
    assert np.all(m == 2.5) and np.all(d == 777.0)


def test_moments_large_offset():
    """x = 1000 + N(0, 1) in float32: the one-pass sum-of-squares formula would lose
    nearly every digit of M2 here; the pairwise merges keep it."""
    x = (random_tensor((40, 5000), 51, torch.float32) + 1000.0)
    mean, m2 = run(fa.fa_moments, x, 1)
    check_moments(x, mean, m2, "offset 1000")
    _, _, m2_ref = oracle.moments(x)
    assert np.max(np.abs(m2 - m2_ref) / m2_ref) < 1e-2


def test_moments_closed_forms():
    x = torch.arange(1, 1025, dtype=torch.float32).repeat(3, 1)
    mean, m2 = run(fa.fa_moments, x, 3)
    assert np.all(mean == 512.5)
    np.testing.assert_allclose(m2, 1024 * (1024 ** 2 - 1) / 12, rtol=1e-6)
    c = torch.full((4, 999), -7.25, dtype=torch.bfloat16)
    mean, m2 = run(fa.fa_moments, c)
    assert np.all(mean == -7.25) and np.all(m2 == 0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", sorted(ROW_WORKLOADS))
def test_full_size_workload_all_rows(name):
    """The benchmark's launches at full size (1 GiB each); every row against the oracle,
    with the tolerances above, the oracle run over blocks of 1024 rows in parallel."""
    w = ROW_WORKLOADS[name]
    x = make_rows(w)
    xd = x.cuda()
    a = torch.empty(w.rows, device="cuda")
    b = torch.empty(w.rows, device="cuda")
    softmax = name.startswith("softmax")
    (fa.fa_softmax_stats if softmax else fa.fa_moments)(xd, a, b)
    torch.cuda.synchronize()
    ga, gb = a.cpu().double().numpy(), b.cpu().double().numpy()
    del xd
    n = w.n
    k = n / 64 + 32

    def block(r0):
        r1 = min(w.rows, r0 + 1024)
        sub = x[r0:r1]
        if softmax:
            m_ref, d_ref = oracle.softmax_stats(sub)
            exact_m = bool(np.array_equal(ga[r0:r1], m_ref))
            rel = float(np.max(np.abs(gb[r0:r1] - d_ref) / d_ref))
            return exact_m, rel / (k * 2 * U)
        _, mu_ref, m2_ref = oracle.moments(sub)
        xa = np.abs(sub.double().numpy()).max(axis=1)
        r_mu = float(np.max(np.abs(ga[r0:r1] - mu_ref) / (k * 2 * U * xa)))
        sigma = np.sqrt(m2_ref / n)
        r_m2 = float(np.max(np.abs(gb[r0:r1] - m2_ref) / m2_ref / (k * 4 * U * xa / sigma)))
        return True, max(r_mu, r_m2)

    res = parallel_map(block, range(0, w.rows, 1024))
    worst = max(r[1] for r in res)
    say(f"{name}: all {w.rows} rows, worst error {worst:.3f} x tolerance")
    assert all(r[0] for r in res), f"{name}: m is not the exact row maximum"
    assert worst <= 1.0, f"{name}: {worst} x tolerance"
