"""fa_decode_noalloc (partial states in the library's static scratch) against the two
calls with caller scratch, fa_decode_partials + fa_combine_partials, through the C ABI.

Two calls in a row on one stream, the second smaller than the first, so the second
reads only states it wrote itself (the array keeps the first call's contents). Both
paths run the same kernels, so their outputs must agree bit for bit; both are also
checked against the fp64 oracle to the decode tolerances (2e-2 bf16 / 1e-4 fp32 on O,
1e-3 on lse).
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


def with_caller_scratch(q, k, v, scale, splits):
    B, H, L, D = k.shape
    m = torch.full((B * H, splits), float("nan"), device="cuda")
    d = torch.full((B * H, splits), float("nan"), device="cuda")
    op = torch.full((B * H, splits, D), float("nan"), device="cuda")
    o = torch.full((B * H, D), float("nan"), device="cuda")
    lse = torch.full((B * H,), float("nan"), device="cuda")
    fa.fa_decode_partials(q, k, v, m, d, op, scale, splits)
    fa.fa_combine_partials(m, d, op, o, lse)
    return o, lse


def without_allocation(q, k, v, scale, splits):
    B, H, L, D = k.shape
    o = torch.full((B * H, D), float("nan"), device="cuda")
    lse = torch.full((B * H,), float("nan"), device="cuda")
    fa.fa_decode_noalloc(q, k, v, o, lse, scale, splits)
    return o, lse


CASES = [
    # (dtype, B, H, L, D, splits): the second of each pair is smaller than the first
    [(torch.bfloat16, 4, 8, 5000, 128, 16), (torch.bfloat16, 2, 3, 700, 64, 5)],
    [(torch.float32, 3, 5, 3001, 64, 7), (torch.float32, 1, 2, 129, 128, 2)],
    [(torch.bfloat16, 16, 32, 4096, 128, 64), (torch.bfloat16, 1, 1, 33, 128, 8)],
]


@pytest.mark.parametrize("pair", CASES, ids=["bf16", "fp32", "wide"])
def test_noalloc_matches_caller_scratch_twice(pair):
    assert torch.cuda.is_available()
    fa.load()
    for call, (dtype, B, H, L, D, splits) in enumerate(pair):
        print(f"noalloc call {call}: dtype={dtype} B={B} H={H} L={L} D={D} splits={splits}",
              flush=True)
        seed = 17 * L + 3 * splits + D + call
        q = random_tensor((B, H, 1, D), seed, dtype)
        k = random_tensor((B, H, L, D), seed + 1, dtype, sigma=2.0)
        v = random_tensor((B, H, L, D), seed + 2, dtype)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        scale = 1 / math.sqrt(D)
        o_ref_gpu, l_ref_gpu = with_caller_scratch(qd, kd, vd, scale, splits)
        o, lse = without_allocation(qd, kd, vd, scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref_gpu), "outputs differ from the caller-scratch path"
        assert torch.equal(lse, l_ref_gpu)
        o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
        eo = float(np.max(np.abs(o.cpu().double().numpy() - o_ref.reshape(B * H, D))))
        el = float(np.max(np.abs(lse.cpu().double().numpy() - lse_ref.reshape(B * H))))
        print(f"  max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
        assert eo <= TOL_O[dtype] and el <= 1e-3


def test_noalloc_rejects_oversize_before_launch():
    fa.load()
    q = torch.zeros(16, 32, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(16, 32, 8, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full((512, 128), 5.0, device="cuda")
    lse = torch.full((512,), 5.0, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_noalloc(q, k, k, o, lse, 0.1, 1024)  # 512 x 1024 units: beyond the array
    assert e.value.code == -7
    torch.cuda.synchronize()
    assert torch.all(o == 5.0) and torch.all(lse == 5.0)


def test_noalloc_no_keys_and_no_torch_allocation():
    """L = 0 writes o = 0, lse = -inf; and the call leaves torch's allocator untouched."""
    fa.load()
    q = random_tensor((2, 2, 1, 64), 5).cuda()
    k = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.full((4, 64), float("nan"), device="cuda")
    lse = torch.full((4,), float("nan"), device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.fa_decode_noalloc(q, k, k, o, lse, 0.125, 3)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
