"""Parity of the prefix scans (fa_softmax_scan, fa_moments_scan, through the C ABI) with
the fp64 oracle, on one MI355X.

Tolerances, from the kernel's float32 arithmetic (u = 2^-24): the state written at
position j is the end of a chain of at most 8 (a lane's own elements) + 6 (the scan
across a wavefront) + 1 (the lanes before) + 4 (the wavefront totals) + n / 2048 (the
carry from earlier blocks) + 2 combines, each a few roundings (one hardware exp2 per
rescale). Hence
* m: exact (a running maximum of the inputs);
* d: relative (n / 2048 + 32) * 4u;
* mean: absolute (n / 2048 + 32) * 4u * max|x|;
* M2: absolute (n / 2048 + 32) * 8u * (j + 1) * max|x|^2 (every merge term of a prefix of
  j + 1 elements is at most (j + 1) max|x|^2).
Rows start on and off 16-byte boundaries and n takes values around the 2048-element
block, so the vector and the per-element paths and the carry between blocks all run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import parallel_map
from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import random_tensor

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


def run(fn, x, offset=0):
    rows, n = x.shape
    buf = torch.full((rows * n + offset + 8,), float("nan"), dtype=x.dtype, device="cuda")
    xd = buf[offset:offset + rows * n].view(rows, n)
    xd.copy_(x.cuda())
    outs = [torch.full((rows * n + offset + 8,), float("nan"), device="cuda") for _ in range(2)]
    a, b = (o[offset:offset + rows * n].view(rows, n) for o in outs)
    fn(xd, a, b)
    torch.cuda.synchronize()
    return a.cpu().double().numpy(), b.cpu().double().numpy()


def check_softmax_scan(x, m, d, what):
    m_ref, d_ref = oracle.softmax_stats_scan(x)
    n = x.shape[1]
    assert np.array_equal(m, m_ref), f"{what}: m is not the exact running maximum"
    live = d_ref > 0
    assert np.all(d[~live] == 0), f"{what}: identity prefixes"
    err = float(np.max(np.abs(d[live] - d_ref[live]) / d_ref[live])) if live.any() else 0.0
    tol = (n / 2048 + 32) * 4 * U
    say(f"{what}: max rel err d {err:.3e} (tol {tol:.3e})")
    assert err <= tol


def check_moments_scan(x, mean, m2, what):
    mu_ref, m2_ref = oracle.moments_scan(x)
    n = x.shape[1]
    xa = np.abs(x.double().numpy()).max(axis=1, keepdims=True)
    k = n / 2048 + 32
    err_mu = np.abs(mean - mu_ref)
    assert np.all(err_mu <= k * 4 * U * xa), f"{what}: mean"
    j1 = np.arange(1, n + 1)[None, :]
    err_m2 = np.abs(m2 - m2_ref)
    say(f"{what}: max |dmean| {err_mu.max():.3e}, max |dM2| {err_m2.max():.3e}")
    assert np.all(err_m2 <= k * 8 * U * j1 * xa ** 2), f"{what}: M2"


SIZES = [1, 7, 8, 9, 100, 2047, 2048, 2049, 5000]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 3])
def test_softmax_scan(dtype, n, offset):
    x = random_tensor((5, n), 700 + n + offset, dtype, sigma=8.0)
    say(f"softmax_scan n={n} {dtype} offset={offset}")
    m, d = run(fa.fa_softmax_scan, x, offset)
    check_softmax_scan(x, m, d, f"softmax_scan n={n} off={offset}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 5])
def test_moments_scan(dtype, n, offset):
    x = random_tensor((5, n), 800 + n + offset, dtype, sigma=2.0) + 1.0
    say(f"moments_scan n={n} {dtype} offset={offset}")
    mean, m2 = run(fa.fa_moments_scan, x, offset)
    check_moments_scan(x, mean, m2, f"moments_scan n={n} off={offset}")


def run_ws(fn, x, offset=0, max_polls=0, workspace=None):
    """As run(), through the workspace entry point (several workgroups per row when the
    row has 2 to 64 whole 2048-element blocks and the tensors are aligned)."""
    rows, n = x.shape
    buf = torch.full((rows * n + offset + 8,), float("nan"), dtype=x.dtype, device="cuda")
    xd = buf[offset:offset + rows * n].view(rows, n)
    xd.copy_(x.cuda())
    outs = [torch.full((rows * n + offset + 8,), float("nan"), device="cuda") for _ in range(2)]
    a, b = (o[offset:offset + rows * n].view(rows, n) for o in outs)
    if workspace is None:
        workspace = torch.empty(max(fa.fa_scan_workspace_bytes(rows, n, x.dtype), 8), dtype=torch.uint8,
                                device="cuda")
    fn(xd, a, b, workspace, max_polls)
    torch.cuda.synchronize()
    return a.cpu().double().numpy(), b.cpu().double().numpy()


# Rows of more than 32 KB with 2 to 64 whole blocks take the chained path when aligned
# (float32: 5 blocks and up; bfloat16: 9 and up); shorter rows, 65 blocks, a ragged
# length or an unaligned row take the one-workgroup-per-row path.
CHAIN_CASES = [(torch.float32, 5 * 2048, 3), (torch.float32, 16384, 2), (torch.float32, 32768, 1),
               (torch.float32, 8192, 3), (torch.bfloat16, 9 * 2048, 2),
               (torch.bfloat16, 32768, 1), (torch.bfloat16, 16384, 2),
               (torch.float32, 20000, 2)]


@pytest.mark.parametrize("dtype,n,rows", CHAIN_CASES,
                         ids=[f"{'bf16' if d == torch.bfloat16 else 'fp32'}-{n}" for d, n, _ in CHAIN_CASES])
@pytest.mark.parametrize("offset", [0, 3])
def test_chained_scans(dtype, n, rows, offset):
    say(f"chained scans n={n} rows={rows} {dtype} offset={offset}")
    x = random_tensor((rows, n), 950 + n + offset, dtype, sigma=8.0)
    m, d = run_ws(fa.fa_softmax_scan_ws, x, offset)
    check_softmax_scan(x, m, d, f"softmax_scan_ws n={n} off={offset}")
    x = random_tensor((rows, n), 960 + n + offset, dtype, sigma=2.0) + 1.0
    mean, m2 = run_ws(fa.fa_moments_scan_ws, x, offset)
    check_moments_scan(x, mean, m2, f"moments_scan_ws n={n} off={offset}")


@pytest.mark.parametrize("polls", [1, 2])
def test_chained_scans_fold_late_blocks_themselves(polls):
    """With one or two polls most blocks find some earlier block's word not yet written
    and fold that block from its elements instead: the results stay within bounds."""
    say(f"chained scans, max_polls={polls}")
    for dtype, n in ((torch.float32, 16384), (torch.bfloat16, 18432)):
        x = random_tensor((3, n), 970 + polls, dtype, sigma=8.0)
        x[1, :3000] = -math.inf
        m, d = run_ws(fa.fa_softmax_scan_ws, x, 0, polls)
        check_softmax_scan(x, m, d, f"softmax_scan_ws polls={polls} {dtype}")
        x = random_tensor((3, n), 980 + polls, dtype, sigma=2.0) + 1.0
        mean, m2 = run_ws(fa.fa_moments_scan_ws, x, 0, polls)
        check_moments_scan(x, mean, m2, f"moments_scan_ws polls={polls} {dtype}")


def test_chained_scans_reuse_one_workspace():
    """Three calls in a row share a workspace: each clears it first, so words left by the
    previous call are never taken for this call's."""
    ws = torch.empty(fa.fa_scan_workspace_bytes(4, 16384), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    for i in range(3):
        x = random_tensor((4, 16384), 990 + i, torch.float32, sigma=4.0 * (i + 1))
        m, d = run_ws(fa.fa_softmax_scan_ws, x, workspace=ws)
        check_softmax_scan(x, m, d, f"softmax_scan_ws call {i}")


def test_softmax_scan_leading_masked_entries():
    """-inf prefixes are the identity; the first finite entry starts d at 1."""
    x = random_tensor((3, 3000), 901, torch.float32, sigma=50.0)
    x[:, :37] = -math.inf
    x[1, 2100:2200] = -math.inf
    m, d = run(fa.fa_softmax_scan, x)
    assert np.all(m[:, :37] == -math.inf) and np.all(d[:, :37] == 0) and np.all(d[:, 37] == 1.0)
    check_softmax_scan(x, m, d, "masked prefixes")


def test_scans_end_in_the_reductions():
    """The last position of each scan is the row reduction of the same rows."""
    x = random_tensor((64, 4100), 902, torch.bfloat16, sigma=3.0)
    m, d = run(fa.fa_softmax_scan, x)
    mean, m2 = run(fa.fa_moments_scan, x)
    xd = x.cuda()
    mr, dr = fa.softmax_stats(xd)
    mur, m2r = fa.moments(xd)
    torch.cuda.synchronize()
    assert np.array_equal(m[:, -1], mr.cpu().double().numpy())
    np.testing.assert_allclose(d[:, -1], dr.cpu().double().numpy(), rtol=1e-5)
    np.testing.assert_allclose(mean[:, -1], mur.cpu().double().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(m2[:, -1], m2r.cpu().double().numpy(), rtol=1e-4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("chained", [False, True], ids=["row_per_workgroup", "chained"])
@pytest.mark.parametrize("name", ["moments_activations_bf16", "softmax_stats_logits_fp32"])
def test_scan_full_size_whole_rows(name, chained):
    """The benchmark's scans at full size (the row reductions' 1 GiB inputs): every
    position of 6 whole rows (the first, the last and 4 seeded ones) against the
    oracle's reduction of each prefix, within the tolerances above; every row's last
    position against the oracle's reduction of the whole row."""
    from exact_io_aware_22_amd.workloads import ROW_WORKLOADS, make_rows

    w = ROW_WORKLOADS[name]
    x = make_rows(w)
    xd = x.cuda()
    a = torch.empty(w.rows, w.n, device="cuda")
    b = torch.empty(w.rows, w.n, device="cuda")
    softmax = name.startswith("softmax")
    say(f"{name} scan at full size, chained={chained}")
    if chained:
        ws = torch.empty(max(fa.fa_scan_workspace_bytes(w.rows, w.n, x.dtype), 8), dtype=torch.uint8,
                         device="cuda")
        (fa.fa_softmax_scan_ws if softmax else fa.fa_moments_scan_ws)(xd, a, b, ws)
    else:
        (fa.fa_softmax_scan if softmax else fa.fa_moments_scan)(xd, a, b)
    torch.cuda.synchronize()
    del xd
    rng = np.random.default_rng(6)
    rows = sorted({0, w.rows - 1, *(int(r) for r in rng.choice(w.rows, 4, replace=False))})
    ga = a[rows].cpu().double().numpy()
    gb = b[rows].cpu().double().numpy()
    last_a = a[:, -1].cpu().double().numpy()
    last_b = b[:, -1].cpu().double().numpy()
    del a, b
    torch.cuda.empty_cache()

    def whole_row(i):
        r = rows[i]
        sub = x[r:r + 1]
        if softmax:
            check_softmax_scan(sub, ga[i:i + 1], gb[i:i + 1], f"{name} row {r} (all {w.n})")
        else:
            check_moments_scan(sub, ga[i:i + 1], gb[i:i + 1], f"{name} row {r} (all {w.n})")

    parallel_map(whole_row, range(len(rows)))
    k = w.n / 2048 + 32
    if softmax:
        m_ref, d_ref = oracle.softmax_stats(x)
        assert np.array_equal(last_a, m_ref)
        assert np.all(np.abs(last_b - d_ref) <= k * 4 * U * d_ref)
    else:
        _, mu_ref, m2_ref = oracle.moments(x)
        xa = x.abs().amax(dim=1).double().numpy()
        assert np.all(np.abs(last_a - mu_ref) <= k * 4 * U * xa)
        assert np.all(np.abs(last_b - m2_ref) <= k * 8 * U * w.n * xa ** 2)
