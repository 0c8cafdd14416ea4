"""Host-side checks of libfa.so: it loads, exports every call include/fa.h declares,
and rejects bad arguments with the documented codes before touching the GPU.

Nothing here launches a kernel: every call either fails validation or describes an
empty problem, both of which return before any HIP call.
"""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

from exact_io_aware_22_amd import fa

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fa.h"

OK, NULL, SHAPE, DTYPE, ALIGN, HIP, ARG, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
P = 1 << 20  # a fake, 16-byte-aligned, never dereferenced address


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not fa._LIB_PATH.exists():
        pytest.fail("libfa.so is not built (python -m exact_io_aware_22_amd.build)")
    return fa.load()


def test_header_declares_the_documented_calls():
    assert declared_functions() == sorted(
        ["fa_forward", "fa_forward_ext", "fa_decode_partials", "fa_combine_partials",
         "fa_decode_noalloc",
         "fa_backward", "fa_softmax_stats", "fa_moments", "fa_softmax_scan", "fa_moments_scan",
         "fa_softmax_scan_ws", "fa_moments_scan_ws", "fa_scan_workspace_bytes",
         "fa_calibrate_mfma", "fa_calibrate_overlap", "fa_calibrate_read", "fa_calibrate_write", "fa_calibrate_mix",
         "fa_strerror", "fa_abi_version"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(fa._LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(fa.EXPORTED) == set(declared_functions())


def test_abi_version_and_strerror(lib):
    assert lib.fa_abi_version() == 2
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, HIP, ARG, SCRATCH, 12345):
        msg = fa.strerror(code)
        assert isinstance(msg, str) and msg


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=8, D=64, scale=0.125, causal=0, dtype=1):
    return lib.fa_forward(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, None)


def test_forward_validation(lib):
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, lse=None) == NULL
    assert fwd(lib, N=-1) == SHAPE
    assert fwd(lib, B=-3) == SHAPE
    assert fwd(lib, D=96) == SHAPE
    assert fwd(lib, D=256) == SHAPE
    assert fwd(lib, B=1 << 30, H=1 << 30, N=1 << 30) == SHAPE
    assert fwd(lib, dtype=7) == DTYPE
    assert fwd(lib, q=P + 8) == ALIGN
    assert fwd(lib, o=P + 4) == ALIGN
    assert fwd(lib, lse=P + 2) == ALIGN
    assert fwd(lib, scale=0.0) == ARG
    assert fwd(lib, scale=-1.0) == ARG
    assert fwd(lib, scale=float("nan")) == ARG
    assert fwd(lib, scale=float("inf")) == ARG
    assert fwd(lib, causal=2) == ARG
    # empty problems are valid and launch nothing
    assert fwd(lib, B=0) == OK
    assert fwd(lib, N=0) == OK
    assert fwd(lib, H=0, D=128, dtype=0) == OK
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, N=0) == OK  # empty tensors
    assert fwd(lib, N=0, D=80) == SHAPE  # sizes are still checked first


def fwx(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=8, D=64, scale=0.125, causal=0, wl=-1,
        wr=-1, cu=None, max_seqlen=0, dtype=1):
    return lib.fa_forward_ext(q, k, v, o, lse, B, H, N, D, scale, causal, wl, wr, cu,
                              max_seqlen, dtype, None)


def test_forward_ext_validation(lib):
    for wl, wr in ((-2, -1), (-1, -7), (-5, 3)):
        assert fwx(lib, wl=wl, wr=wr) == ARG
    assert fwx(lib, wl=3, dtype=0) == DTYPE  # windows need bf16
    assert fwx(lib, cu=P, max_seqlen=8, dtype=0) == DTYPE  # packed needs bf16
    assert fwx(lib, cu=P, max_seqlen=-1) == SHAPE
    assert fwx(lib, cu=P + 2, max_seqlen=8) == ALIGN
    assert fwx(lib, cu=P, max_seqlen=8, lse=None) == NULL
    assert fwx(lib, wl=4, wr=0, q=P + 8) == ALIGN
    # packed size check is on H x N x D: B counts sequences and may be large
    assert fwx(lib, B=1 << 30, H=4, N=1 << 10, cu=P, max_seqlen=0) == OK
    assert fwx(lib, B=1 << 30, H=1 << 30, N=1 << 30) == SHAPE
    # empty problems: no pointer is touched
    assert fwx(lib, cu=P, max_seqlen=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert fwx(lib, N=0, wl=5, q=None) == OK
    assert fwx(lib, B=0, cu=P, max_seqlen=4) == OK  # no sequences
    assert fwx(lib, N=0, D=72) == SHAPE


def dec(lib, q=P, k=P, v=P, m=P, d=P, op=P, B=1, H=1, L=64, D=128, scale=0.1, splits=4, dtype=1):
    return lib.fa_decode_partials(q, k, v, m, d, op, B, H, L, D, scale, splits, dtype, None)


def test_decode_validation(lib):
    assert dec(lib, m=None) == NULL
    assert dec(lib, splits=0) == SHAPE
    assert dec(lib, L=-1) == SHAPE
    assert dec(lib, D=32) == SHAPE
    assert dec(lib, dtype=-1) == DTYPE
    assert dec(lib, k=P + 4) == ALIGN
    assert dec(lib, op=P + 8) == ALIGN
    assert dec(lib, m=P + 1) == ALIGN
    assert dec(lib, scale=0.0) == ARG
    assert dec(lib, B=0) == OK
    assert dec(lib, H=0) == OK
    assert dec(lib, q=None, B=0) == OK
    assert dec(lib, q=None, L=0) == NULL  # L = 0 is not empty: it writes identities


def comb(lib, m=P, d=P, op=P, splits=4, rows=3, D=64, o=P, lse=P):
    return lib.fa_combine_partials(m, d, op, splits, rows, D, o, lse, None)


def test_combine_validation(lib):
    assert comb(lib, o=None) == NULL
    assert comb(lib, splits=0) == SHAPE
    assert comb(lib, rows=-1) == SHAPE
    assert comb(lib, D=100) == SHAPE
    assert comb(lib, op=P + 4) == ALIGN
    assert comb(lib, lse=P + 1) == ALIGN
    assert comb(lib, rows=0) == OK
    assert comb(lib, rows=0, m=None, o=None) == OK


def bwd(lib, q=P, k=P, v=P, o=P, lse=P, do=P, delta=P, dq=P, dk=P, dv=P, B=1, H=2, N=8, D=128,
        scale=0.1, causal=1, dtype=1):
    return lib.fa_backward(q, k, v, o, lse, do, delta, dq, dk, dv, B, H, N, D, scale, causal,
                           dtype, None)


def test_backward_validation(lib):
    for name in ("q", "k", "v", "o", "lse", "do", "delta", "dq", "dk", "dv"):
        assert bwd(lib, **{name: None}) == NULL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwd(lib, **{name: P + 8}) == ALIGN, name
    assert bwd(lib, lse=P + 2) == ALIGN
    assert bwd(lib, delta=P + 1) == ALIGN
    assert bwd(lib, N=-1) == SHAPE
    assert bwd(lib, D=48) == SHAPE
    assert bwd(lib, dtype=2) == DTYPE
    assert bwd(lib, scale=0.0) == ARG
    assert bwd(lib, causal=-1) == ARG
    assert bwd(lib, B=0) == OK
    assert bwd(lib, N=0, q=None, dq=None, delta=None) == OK
    assert bwd(lib, N=0, D=40) == SHAPE


def test_binding_raises_with_message(lib):
    with pytest.raises(fa.FaError, match="scale"):
        fa._check(lib.fa_forward(P, P, P, P, P, 1, 1, 8, 64, -1.0, 0, 1, None), "fa_forward")


def red(lib, which, x=P, o0=P, o1=P, rows=4, n=100, dtype=1):
    return getattr(lib, which)(x, o0, o1, rows, n, dtype, None)


@pytest.mark.parametrize("which", ["fa_softmax_stats", "fa_moments"])
def test_row_reduction_validation(lib, which):
    assert red(lib, which, x=None) == NULL
    assert red(lib, which, o0=None) == NULL
    assert red(lib, which, o1=None) == NULL
    assert red(lib, which, rows=-1) == SHAPE
    assert red(lib, which, n=-5) == SHAPE
    assert red(lib, which, dtype=3) == DTYPE
    assert red(lib, which, x=P + 1) == ALIGN          # bf16 needs 2-byte alignment
    assert red(lib, which, x=P + 2, dtype=0) == ALIGN  # fp32 needs 4
    assert red(lib, which, o1=P + 2) == ALIGN
    assert red(lib, which, rows=0, x=None, o0=None, o1=None) == OK  # empty
    assert red(lib, which, rows=0, n=-1) == SHAPE                    # sizes first


@pytest.mark.parametrize("which", ["fa_softmax_scan", "fa_moments_scan"])
def test_row_scan_validation(lib, which):
    assert red(lib, which, x=None) == NULL
    assert red(lib, which, o1=None) == NULL
    assert red(lib, which, rows=-1) == SHAPE
    assert red(lib, which, n=-1) == SHAPE
    assert red(lib, which, dtype=5) == DTYPE
    assert red(lib, which, x=P + 1) == ALIGN
    assert red(lib, which, x=P + 2, dtype=0) == ALIGN
    assert red(lib, which, o0=P + 3) == ALIGN
    assert red(lib, which, rows=0, x=None, o0=None, o1=None) == OK  # empty
    assert red(lib, which, n=0, x=None, o0=None, o1=None) == OK     # empty rows
    assert red(lib, which, rows=1 << 30, n=1 << 30) == SHAPE         # offsets overflow


def test_scan_workspace_bytes(lib):
    f = lib.fa_scan_workspace_bytes
    F32, BF16 = 0, 1
    assert f(8192, 32768, F32) == 8192 * 16 * 8  # 16 blocks of 2048 per 128 KB row
    assert f(65536, 8192, BF16) == 0             # 16 KB rows: one workgroup each
    assert f(3, 5 * 2048, F32) == 3 * 5 * 8      # 40 KB rows: cut
    assert f(3, 4 * 2048, F32) == 0              # 32 KB rows: not
    assert f(3, 9 * 2048, BF16) == 3 * 9 * 8
    assert f(3, 8 * 2048, BF16) == 0
    assert f(3, 64 * 2048, BF16) == 3 * 64 * 8   # the most blocks that are cut
    for n in (0, 1, 2047, 2048, 6000, 65 * 2048, 20000):
        assert f(5, n, F32) == 0, n              # one workgroup per row
    assert f(0, 32768, F32) == 0
    assert f(-1, 4096, F32) == -1 and f(5, -1, F32) == -1 and f(5, 32768, 7) == -1
    assert f(1 << 30, 1 << 30, F32) == -1        # offsets overflow


@pytest.mark.parametrize("which", ["fa_softmax_scan_ws", "fa_moments_scan_ws"])
def test_row_scan_ws_validation(lib, which):
    fn = getattr(lib, which)

    def call(x=P, o0=P, o1=P, rows=4, n=32768, dtype=1, ws=P, nbytes=4 * 16 * 8, polls=0):
        return fn(x, o0, o1, rows, n, dtype, ws, nbytes, polls, None)

    assert call(x=None) == NULL
    assert call(ws=None) == NULL                  # 16 blocks per row: the workspace is needed
    assert call(nbytes=4 * 16 * 8 - 1) == SCRATCH
    assert call(ws=P + 4) == ALIGN
    assert call(polls=-1) == ARG
    assert call(rows=-1) == SHAPE
    assert call(dtype=7) == DTYPE
    assert call(x=P + 1) == ALIGN
    assert call(rows=0, x=None, o0=None, o1=None, ws=None, nbytes=0) == OK  # empty
    assert call(n=0, x=None, o0=None, o1=None, ws=None, nbytes=0) == OK     # empty rows


def test_calibration_validation(lib):
    mf, rd = lib.fa_calibrate_mfma, lib.fa_calibrate_read
    assert mf(None, 4, 1, 0, None) == NULL
    assert mf(P, 0, 1, 0, None) == SHAPE
    assert mf(P, (1 << 20) + 1, 1, 0, None) == SHAPE
    assert mf(P, 4, -1, 0, None) == SHAPE
    assert mf(P + 2, 4, 1, 0, None) == ALIGN
    assert rd(P, 1024, None, 4, None) == NULL
    assert rd(None, 1024, P, 4, None) == NULL
    assert rd(P, 1000, P, 4, None) == SHAPE   # not a multiple of 16
    assert rd(P, -16, P, 4, None) == SHAPE
    assert rd(P, 1024, P, 0, None) == SHAPE
    assert rd(P + 8, 1024, P, 4, None) == ALIGN
    assert rd(P, 1024, P + 1, 4, None) == ALIGN
    wr = lib.fa_calibrate_write
    assert wr(None, 1024, 1, 4, None) == NULL
    assert wr(None, 0, 1, 4, None) == OK     # empty: returns before any HIP call
    assert wr(P, 1000, 1, 4, None) == SHAPE
    assert wr(P, 1024, 1, 0, None) == SHAPE
    assert wr(P + 8, 1024, 1, 4, None) == ALIGN
    mx = lib.fa_calibrate_mix
    assert mx(None, 0, None, 1, 4, None) == OK      # empty: returns before any HIP call
    assert mx(None, 4096, P, 1, 4, None) == NULL
    assert mx(P, 4096, None, 2, 4, None) == NULL
    assert mx(P, 4000, P, 1, 4, None) == SHAPE      # not a multiple of 4096
    assert mx(P, 2048, P, 1, 4, None) == SHAPE
    assert mx(P, -4096, P, 1, 4, None) == SHAPE
    assert mx(P, 4096, P, 3, 4, None) == SHAPE      # ratio 1, 2 or 4 only
    assert mx(P, 4096, P, 0, 4, None) == SHAPE
    assert mx(P, 4096, P, 1, 0, None) == SHAPE
    assert mx(P, 4096, P, 1, (1 << 22) + 1, None) == SHAPE
    assert mx(P + 8, 4096, P, 1, 4, None) == ALIGN
    assert mx(P, 4096, P + 4, 1, 4, None) == ALIGN



SCRATCH_FLOATS = 8388608


def dec_noalloc(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=2, L=64, D=128, scale=0.1, splits=4,
                dtype=1):
    return lib.fa_decode_noalloc(q, k, v, o, lse, B, H, L, D, scale, splits, dtype, None)


def test_decode_noalloc_validation(lib):
    header = HEADER.read_text()
    assert f"#define FA_DECODE_SCRATCH_FLOATS {SCRATCH_FLOATS}" in header
    assert dec_noalloc(lib, splits=0) == SHAPE
    assert dec_noalloc(lib, D=96) == SHAPE
    assert dec_noalloc(lib, L=-1) == SHAPE
    assert dec_noalloc(lib, dtype=3) == DTYPE
    assert dec_noalloc(lib, scale=0.0) == ARG
    assert dec_noalloc(lib, q=None) == NULL
    assert dec_noalloc(lib, lse=None) == NULL
    assert dec_noalloc(lib, o=P + 4) == ALIGN
    assert dec_noalloc(lib, B=0) == OK and dec_noalloc(lib, H=0, q=None) == OK
    # the limit: 2 * ceil64(R) + R * D floats, R = B * H * splits
    def need(R, D):
        return 2 * (-(-R // 64) * 64) + R * D
    assert need(16 * 32 * 64, 128) <= SCRATCH_FLOATS  # the split-KV decode workload fits
    R_max = max(R for R in range(SCRATCH_FLOATS // 130 - 64, SCRATCH_FLOATS // 130 + 64)
                if need(R, 128) <= SCRATCH_FLOATS)
    # R_max units fit; one more does not; checked before any launch, whatever L is
    assert dec_noalloc(lib, B=1, H=1, splits=R_max + 1, L=1 << 20) == SCRATCH
    assert dec_noalloc(lib, B=R_max + 1, H=1, splits=1) == SCRATCH
    assert dec_noalloc(lib, B=16, H=32, splits=1024) == SCRATCH
    assert dec_noalloc(lib, B=16, H=32, splits=1024, D=64, L=0, k=None, v=None) == SCRATCH
    assert dec_noalloc(lib, B=1, H=1, splits=R_max + 1, D=64, q=None) == NULL  # fits at D=64
    assert "static scratch" in fa.strerror(SCRATCH)


def test_library_imports_no_allocator():
    """Nothing in libfa.so allocates device or host memory: no HIP allocation routine
    is even imported (the static scratch of fa_decode_noalloc is a device global)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", str(fa._LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    imported = set(re.findall(r"\bU\s+(\S+?)(?:@\S+)?$", out, flags=re.M))
    allocators = {n for n in imported if re.match(r"hip(Ext)?(Host|Managed)?(Malloc|Free|Alloc)", n)
                  or n.startswith("hipMemPool") or n.startswith("hipMallocAsync")}
    assert not allocators, allocators
    assert "hipGetSymbolAddress" in imported
