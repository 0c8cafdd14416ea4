"""ctypes binding of libfa.so (C ABI in include/fa.h).

Argument marshalling only: torch tensors are passed as raw device pointers plus
sizes, and the current torch stream as the HIP stream. Every step of the
computation runs in the library's HIP kernels. If the library is missing or
cannot be loaded this module raises; there is no other code path.

Functions with the C names (fa_forward, fa_decode_partials, fa_combine_partials)
take caller-allocated outputs, as the C calls do. forward / decode are
conveniences that allocate the outputs with torch and call them.
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path

import torch

_LIB_PATH = Path(os.environ.get("FA_LIB", Path(__file__).resolve().parent / "libfa.so"))
_lib = None

FA_F32, FA_BF16 = 0, 1
_DTYPES = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}
EXPORTED = ("fa_forward", "fa_forward_ext", "fa_decode_partials", "fa_combine_partials",
            "fa_decode_noalloc", "fa_backward", "fa_softmax_stats", "fa_moments",
            "fa_softmax_scan", "fa_moments_scan", "fa_softmax_scan_ws", "fa_moments_scan_ws",
            "fa_scan_workspace_bytes", "fa_calibrate_mfma", "fa_calibrate_overlap",
            "fa_calibrate_read", "fa_calibrate_write", "fa_calibrate_mix", "fa_strerror",
            "fa_abi_version")


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load():
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m exact_io_aware_22_amd.build`")
    lib = ctypes.CDLL(str(_LIB_PATH))
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp, i, i, vp]
    lib.fa_forward_ext.restype = i
    lib.fa_softmax_stats.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.fa_softmax_stats.restype = i
    lib.fa_moments.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.fa_moments.restype = i
    for name in ("fa_softmax_scan", "fa_moments_scan"):
        getattr(lib, name).argtypes = [vp, vp, vp, i, i, i, vp]
        getattr(lib, name).restype = i
    for name in ("fa_softmax_scan_ws", "fa_moments_scan_ws"):
        getattr(lib, name).argtypes = [vp, vp, vp, i, i, i, vp, ctypes.c_longlong, i, vp]
        getattr(lib, name).restype = i
    lib.fa_scan_workspace_bytes.argtypes = [i, i, i]
    lib.fa_scan_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_decode_partials.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_decode_partials.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_combine_partials.argtypes = [vp, vp, vp, i, i, i, vp, vp, vp]
    lib.fa_combine_partials.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_backward.restype = i
    lib.fa_calibrate_mfma.argtypes = [vp, i, i, ctypes.c_uint, vp]
    lib.fa_calibrate_mfma.restype = i
    lib.fa_calibrate_overlap.argtypes = [vp, i, i, i, vp]
    lib.fa_calibrate_overlap.restype = i
    lib.fa_calibrate_read.argtypes = [vp, ctypes.c_longlong, vp, i, vp]
    lib.fa_calibrate_read.restype = i
    lib.fa_calibrate_write.argtypes = [vp, ctypes.c_longlong, ctypes.c_uint, i, vp]
    lib.fa_calibrate_write.restype = i
    lib.fa_calibrate_mix.argtypes = [vp, ctypes.c_longlong, vp, i, i, vp]
    lib.fa_calibrate_mix.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().fa_strerror(int(code)).decode()


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(code: int, where: str):
    if code != 0:
        raise FaError(code, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")
    return _DTYPES[t.dtype]


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# Validation of every tensor a C-named wrapper passes on. The library receives raw
# pointers only, so a tensor of the wrong shape, dtype or device would otherwise be
# read or written out of bounds on the GPU. Checks run in this order, before the
# library is loaded: dtypes, shapes, contiguity, then that every tensor lives on one
# CUDA device.
def _want_dtype(name: str, t: torch.Tensor, dtype: torch.dtype) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _want_shape(name: str, t: torch.Tensor, shape: tuple) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_input_dtype(**ts) -> int:
    """q, k, v (and dout) share one supported dtype; returns its FA_* code."""
    items = list(ts.items())
    code = _dtype_code(items[0][1])
    for name, t in items[1:]:
        if t.dtype != items[0][1].dtype:
            raise TypeError(f"{name} must have the dtype of {items[0][0]} ({items[0][1].dtype}), "
                            f"got {t.dtype}")
    return code


def _on_one_device(**ts) -> None:
    dev = None
    for name, t in ts.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _checked(shapes: dict, f32: tuple, **ts) -> None:
    """Shapes from `shapes` (name -> tuple), float32 for the names in `f32`, then
    contiguity and one CUDA device for every tensor in ts."""
    for name in f32:
        _want_dtype(name, ts[name], torch.float32)
    for name, shape in shapes.items():
        _want_shape(name, ts[name], shape)
    _dense(*ts.values())
    _on_one_device(**ts)


# ------------------------------------------------------------------ C-named calls
def fa_forward(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """q, k, v: [B, H, N, D] (bf16 or fp32, same dtype); o: [B, H, N, D] fp32; lse: [B, H, N] fp32."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, D], got shape {tuple(q.shape)}")
    B, H, N, D = q.shape
    dt = _same_input_dtype(q=q, k=k, v=v)
    _checked({"k": q.shape, "v": q.shape, "o": q.shape, "lse": (B, H, N)}, ("o", "lse"),
             q=q, k=k, v=v, o=o, lse=lse)
    code = load().fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D,
                             float(scale), int(bool(causal)), dt, _stream(stream))
    _check(code, "fa_forward")


def fa_forward_ext(q, k, v, o, lse, scale: float, causal: bool, window_left: int = -1,
                   window_right: int = -1, cu_seqlens=None, max_seqlen: int = 0,
                   stream=None) -> None:
    """Dense: as fa_forward, plus the window. Packed (cu_seqlens, an int32 device tensor
    of nseq + 1 offsets): q, k, v, o [H, total, D], lse [H, total]."""
    if cu_seqlens is not None:
        if q.dim() != 3:
            raise ValueError(f"packed q must be [H, total, D], got shape {tuple(q.shape)}")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
        H, N, D = q.shape
        B = cu_seqlens.numel() - 1
        lse_shape = (H, N)
    else:
        if q.dim() != 4:
            raise ValueError(f"q must be [B, H, N, D], got shape {tuple(q.shape)}")
        B, H, N, D = q.shape
        lse_shape = (B, H, N)
    dt = _same_input_dtype(q=q, k=k, v=v)
    _checked({"k": q.shape, "v": q.shape, "o": q.shape, "lse": lse_shape}, ("o", "lse"),
             q=q, k=k, v=v, o=o, lse=lse, cu_seqlens=cu_seqlens)
    code = load().fa_forward_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D,
                                 float(scale), int(bool(causal)), int(window_left),
                                 int(window_right), _ptr(cu_seqlens), int(max_seqlen),
                                 dt, _stream(stream))
    _check(code, "fa_forward_ext")


def fa_decode_partials(q, k, v, m, d, o_part, scale: float, splits: int, stream=None) -> None:
    """q: [B, H, 1, D] or [B, H, D]; k, v: [B, H, L, D]; m, d: [B*H, splits]; o_part: [B*H, splits, D]."""
    if k.dim() != 4:
        raise ValueError(f"k must be [B, H, L, D], got shape {tuple(k.shape)}")
    B, H, L, D = k.shape
    splits = int(splits)
    if splits < 1:
        raise ValueError("splits must be >= 1")
    if tuple(q.shape) not in ((B, H, 1, D), (B, H, D)):
        raise ValueError(f"q must have shape {(B, H, 1, D)} or {(B, H, D)}, got {tuple(q.shape)}")
    dt = _same_input_dtype(k=k, q=q, v=v)
    _checked({"v": k.shape, "m": (B * H, splits), "d": (B * H, splits),
              "o_part": (B * H, splits, D)}, ("m", "d", "o_part"),
             q=q, k=k, v=v, m=m, d=d, o_part=o_part)
    code = load().fa_decode_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(d), _ptr(o_part),
                                     B, H, L, D, float(scale), splits, dt, _stream(stream))
    _check(code, "fa_decode_partials")


def fa_decode_noalloc(q, k, v, o, lse, scale: float, splits: int, stream=None) -> None:
    """Partials and merge in one call, the partial states in the library's static
    scratch (no allocation). q: [B, H, 1, D] or [B, H, D]; k, v: [B, H, L, D];
    o: [B*H, D] fp32; lse: [B*H] fp32. Calls that overlap on one GPU race on that
    scratch; calls on one stream are ordered."""
    if k.dim() != 4:
        raise ValueError(f"k must be [B, H, L, D], got shape {tuple(k.shape)}")
    B, H, L, D = k.shape
    splits = int(splits)
    if splits < 1:
        raise ValueError("splits must be >= 1")
    if tuple(q.shape) not in ((B, H, 1, D), (B, H, D)):
        raise ValueError(f"q must have shape {(B, H, 1, D)} or {(B, H, D)}, got {tuple(q.shape)}")
    dt = _same_input_dtype(k=k, q=q, v=v)
    _checked({"v": k.shape, "o": (B * H, D), "lse": (B * H,)}, ("o", "lse"),
             q=q, k=k, v=v, o=o, lse=lse)
    code = load().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, L, D,
                                    float(scale), splits, dt, _stream(stream))
    _check(code, "fa_decode_noalloc")


def fa_combine_partials(m, d, o_part, o, lse, stream=None) -> None:
    """m, d: [rows, splits] fp32; o_part: [rows, splits, D] fp32; o: [rows, D]; lse: [rows]."""
    if o_part.dim() != 3:
        raise ValueError(f"o_part must be [rows, splits, D], got shape {tuple(o_part.shape)}")
    rows, splits, D = o_part.shape
    _checked({"m": (rows, splits), "d": (rows, splits), "o": (rows, D), "lse": (rows,)},
             ("m", "d", "o_part", "o", "lse"), m=m, d=d, o_part=o_part, o=o, lse=lse)
    code = load().fa_combine_partials(_ptr(m), _ptr(d), _ptr(o_part), splits, rows, D,
                                      _ptr(o), _ptr(lse), _stream(stream))
    _check(code, "fa_combine_partials")


def fa_backward(q, k, v, o, lse, dout, delta, dq, dk, dv, scale: float, causal: bool,
                stream=None) -> None:
    """q, k, v, dout: [B, H, N, D] (bf16 or fp32, same dtype); o: [B, H, N, D] fp32 and
    lse: [B, H, N] fp32 from fa_forward; delta: [B, H, N] fp32 scratch; dq, dk, dv:
    [B, H, N, D] fp32, written."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, D], got shape {tuple(q.shape)}")
    B, H, N, D = q.shape
    dt = _same_input_dtype(q=q, k=k, v=v, dout=dout)
    s = tuple(q.shape)
    _checked({"k": s, "v": s, "dout": s, "o": s, "dq": s, "dk": s, "dv": s, "lse": (B, H, N),
              "delta": (B, H, N)}, ("o", "lse", "delta", "dq", "dk", "dv"),
             q=q, k=k, v=v, o=o, lse=lse, dout=dout, delta=delta, dq=dq, dk=dk, dv=dv)
    code = load().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                              _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, D,
                              float(scale), int(bool(causal)), dt, _stream(stream))
    _check(code, "fa_backward")


def _rows(x, out0, out1):
    if x.dim() < 1:
        raise ValueError("x needs at least one dimension (its rows are along the last)")
    _dtype_code(x)
    n, rows = x.shape[-1], math.prod(x.shape[:-1])
    for name, t in (("out0", out0), ("out1", out1)):
        _want_dtype(name, t, torch.float32)
        if t.numel() != rows:
            raise ValueError(f"outputs must hold one value per row ({rows})")
    _dense(x, out0, out1)
    _on_one_device(x=x, out0=out0, out1=out1)
    return rows, n


def fa_softmax_stats(x, m, d, stream=None) -> None:
    """x: [..., n] (bf16 or fp32); m, d: fp32 with one element per row of x."""
    rows, n = _rows(x, m, d)
    code = load().fa_softmax_stats(_ptr(x), _ptr(m), _ptr(d), rows, n, _dtype_code(x),
                                   _stream(stream))
    _check(code, "fa_softmax_stats")


def fa_moments(x, mean, m2, stream=None) -> None:
    """x: [..., n] (bf16 or fp32); mean, m2: fp32 with one element per row of x."""
    rows, n = _rows(x, mean, m2)
    code = load().fa_moments(_ptr(x), _ptr(mean), _ptr(m2), rows, n, _dtype_code(x),
                             _stream(stream))
    _check(code, "fa_moments")


def _scan_shapes(x, out0, out1):
    if x.dim() < 1:
        raise ValueError("x needs at least one dimension (its rows are along the last)")
    _dtype_code(x)
    for name, t in (("out0", out0), ("out1", out1)):
        _want_dtype(name, t, torch.float32)
        if t.shape != x.shape:
            raise ValueError("scan outputs must have x's shape")
    _dense(x, out0, out1)
    _on_one_device(x=x, out0=out0, out1=out1)
    return math.prod(x.shape[:-1]), x.shape[-1]


def fa_softmax_scan(x, m, d, stream=None) -> None:
    """x: [..., n] (bf16 or fp32); m, d: fp32 of x's shape (inclusive prefix states)."""
    rows, n = _scan_shapes(x, m, d)
    code = load().fa_softmax_scan(_ptr(x), _ptr(m), _ptr(d), rows, n, _dtype_code(x),
                                  _stream(stream))
    _check(code, "fa_softmax_scan")


def fa_moments_scan(x, mean, m2, stream=None) -> None:
    """x: [..., n] (bf16 or fp32); mean, m2: fp32 of x's shape (inclusive prefix moments)."""
    rows, n = _scan_shapes(x, mean, m2)
    code = load().fa_moments_scan(_ptr(x), _ptr(mean), _ptr(m2), rows, n, _dtype_code(x),
                                  _stream(stream))
    _check(code, "fa_moments_scan")


def fa_scan_workspace_bytes(rows: int, n: int, dtype=torch.float32) -> int:
    """Workspace bytes fa_softmax_scan_ws / fa_moments_scan_ws need for rows x n elements
    of dtype (a torch dtype)."""
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}; expected float32 or bfloat16")
    nbytes = load().fa_scan_workspace_bytes(int(rows), int(n), _DTYPES[dtype])
    if nbytes < 0:
        raise ValueError(f"invalid scan size rows={rows} n={n}")
    return int(nbytes)


def _scan_ws(name, x, out0, out1, workspace, max_polls, stream):
    rows, n = _scan_shapes(x, out0, out1)
    need = fa_scan_workspace_bytes(rows, n, x.dtype)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _want_dtype("workspace", workspace, torch.uint8)
        _dense(workspace)
        _on_one_device(x=x, workspace=workspace)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    if ws_bytes < need:
        raise ValueError(f"workspace must hold {need} bytes, got {ws_bytes}")
    code = getattr(load(), name)(_ptr(x), _ptr(out0), _ptr(out1), rows, n, _dtype_code(x),
                                 ws_ptr, ws_bytes, int(max_polls), _stream(stream))
    _check(code, name)


def fa_softmax_scan_ws(x, m, d, workspace, max_polls: int = 0, stream=None) -> None:
    """fa_softmax_scan with a uint8 device workspace of fa_scan_workspace_bytes bytes, which
    lets several workgroups share a row (see include/fa.h)."""
    _scan_ws("fa_softmax_scan_ws", x, m, d, workspace, max_polls, stream)


def fa_moments_scan_ws(x, mean, m2, workspace, max_polls: int = 0, stream=None) -> None:
    """fa_moments_scan with a workspace, as fa_softmax_scan_ws."""
    _scan_ws("fa_moments_scan_ws", x, mean, m2, workspace, max_polls, stream)


def fa_calibrate_mfma(out, blocks: int, iters: int, seed: int = 0, stream=None) -> None:
    """Measurement only: the MFMA-only loop; out: fp32 [blocks * 512] (checksums).
    One launch is 2**19 * 8 * blocks * iters flops."""
    if out.dtype != torch.float32 or out.numel() != blocks * 512:
        raise ValueError("out must be float32 with blocks * 512 elements")
    _dense(out)
    _on_one_device(out=out)
    code = load().fa_calibrate_mfma(_ptr(out), int(blocks), int(iters), int(seed) & 0xFFFFFFFF,
                                    _stream(stream))
    _check(code, "fa_calibrate_mfma")


def fa_calibrate_overlap(out, blocks: int, iters: int, mode: int, stream=None) -> None:
    """Measurement only: the matrix/vector overlap probe (modes 0-6 and 8-13, see
    include/fa.h); out: fp32 [blocks * 512] (checksums, SIMD indices in mode 6, elapsed
    cycles / real-time ticks in modes 8-13)."""
    if out.dtype != torch.float32 or out.numel() != blocks * 512:
        raise ValueError("out must be float32 with blocks * 512 elements")
    _dense(out)
    _on_one_device(out=out)
    code = load().fa_calibrate_overlap(_ptr(out), int(blocks), int(iters), int(mode),
                                       _stream(stream))
    _check(code, "fa_calibrate_overlap")


def fa_calibrate_read(x, out, blocks: int, stream=None) -> None:
    """Measurement only: a read-only stream over the bytes of x (a multiple of 16);
    out: int32 [blocks * 256], each thread's XOR of the 32-bit words it read."""
    if out.dtype != torch.int32 or out.numel() != blocks * 256:
        raise ValueError("out must be int32 with blocks * 256 elements")
    _dense(x, out)
    _on_one_device(x=x, out=out)
    nbytes = x.numel() * x.element_size()
    code = load().fa_calibrate_read(_ptr(x), nbytes, _ptr(out), int(blocks), _stream(stream))
    _check(code, "fa_calibrate_read")


def fa_calibrate_write(y, value: int, blocks: int, stream=None) -> None:
    """Measurement only: a write-only stream over the bytes of y (a multiple of 16);
    16-byte word w becomes {value, w, value, w} as 32-bit words."""
    _dense(y)
    _on_one_device(y=y)
    nbytes = y.numel() * y.element_size()
    code = load().fa_calibrate_write(_ptr(y), nbytes, int(value) & 0xFFFFFFFF, int(blocks),
                                     _stream(stream))
    _check(code, "fa_calibrate_write")


def fa_calibrate_mix(x, y, ratio: int, blocks: int, stream=None) -> None:
    """Measurement only: reads the bytes of x (a multiple of 4096) and writes them to two
    output streams, each `ratio` times as many bytes, in y (at least 2 * ratio times the
    bytes of x): the run of 256 16-byte words at word j goes to words ratio j + 256 r + t
    (word j + t) of both streams."""
    _dense(x, y)
    _on_one_device(x=x, y=y)
    nbytes = x.numel() * x.element_size()
    if y.numel() * y.element_size() < 2 * int(ratio) * nbytes:
        raise ValueError("y must hold 2 * ratio times the bytes of x")
    code = load().fa_calibrate_mix(_ptr(x), nbytes, _ptr(y), int(ratio), int(blocks),
                                   _stream(stream))
    _check(code, "fa_calibrate_mix")


# ------------------------------------------------------------------ conveniences
def softmax_stats(x, stream=None):
    """Allocate m, d (x's shape without its last dim, fp32) and run fa_softmax_stats."""
    m = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    d = torch.empty_like(m)
    fa_softmax_stats(x, m, d, stream)
    return m, d


def _workspace_for(x):
    rows = math.prod(x.shape[:-1]) if x.dim() > 0 else 0
    need = fa_scan_workspace_bytes(rows, x.shape[-1], x.dtype) if x.dim() > 0 else 0
    return torch.empty(max(need, 8), dtype=torch.uint8, device=x.device)


def softmax_scan(x, stream=None):
    """Allocate m, d (x's shape, fp32) and a workspace, and run fa_softmax_scan_ws."""
    m = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    d = torch.empty_like(m)
    fa_softmax_scan_ws(x, m, d, _workspace_for(x), 0, stream)
    return m, d


def moments_scan(x, stream=None):
    """Allocate mean, m2 (x's shape, fp32) and a workspace, and run fa_moments_scan_ws."""
    mean = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    m2 = torch.empty_like(mean)
    fa_moments_scan_ws(x, mean, m2, _workspace_for(x), 0, stream)
    return mean, m2


def moments(x, stream=None):
    """Allocate mean, m2 (x's shape without its last dim, fp32) and run fa_moments."""
    mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    m2 = torch.empty_like(mean)
    fa_moments(x, mean, m2, stream)
    return mean, m2

def forward(q, k, v, scale: float | None = None, causal: bool = False, stream=None):
    """Allocate O [B, H, N, D] fp32 and lse [B, H, N] fp32 and run fa_forward."""
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty(B, H, N, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    fa_forward(q, k, v, o, lse, scale, causal, stream)
    return o, lse


def forward_ext(q, k, v, scale: float | None = None, causal: bool = False,
                window_left: int = -1, window_right: int = -1, cu_seqlens=None,
                max_seqlen: int | None = None, stream=None):
    """Allocate O (q's shape, fp32) and lse (q's shape without D, fp32) and run
    fa_forward_ext. Packed (cu_seqlens given): q, k, v [H, total, D]; max_seqlen
    defaults to the longest sequence (read from cu_seqlens on the host). Rows that no
    sequence covers are left unwritten."""
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if cu_seqlens is not None and max_seqlen is None:
        c = cu_seqlens.cpu()
        max_seqlen = int((c[1:] - c[:-1]).max()) if c.numel() > 1 else 0
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_forward_ext(q, k, v, o, lse, scale, causal, window_left, window_right, cu_seqlens,
                   max_seqlen or 0, stream)
    return o, lse


def backward(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False,
             stream=None):
    """Allocate Delta scratch and dq, dk, dv [B, H, N, D] fp32 and run fa_backward.
    o and lse are the outputs of `forward` for the same q, k, v, scale and causal."""
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = q.device
    delta = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(B, H, N, D, dtype=torch.float32, device=dev) for _ in range(3))
    fa_backward(q, k, v, o, lse, dout, delta, dq, dk, dv, scale, causal, stream)
    return dq, dk, dv


def decode(q, k, v, splits: int, scale: float | None = None, stream=None, return_partials=False):
    """Split-KV decode: partial states per chunk, then their merge. Returns
    (o [B, H, 1, D] fp32, lse [B, H, 1] fp32) and, if asked, the partials."""
    B, H, L, D = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = k.device
    m = torch.empty(B * H, splits, dtype=torch.float32, device=dev)
    d = torch.empty(B * H, splits, dtype=torch.float32, device=dev)
    op = torch.empty(B * H, splits, D, dtype=torch.float32, device=dev)
    o = torch.empty(B * H, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B * H, dtype=torch.float32, device=dev)
    fa_decode_partials(q, k, v, m, d, op, scale, splits, stream)
    fa_combine_partials(m, d, op, o, lse, stream)
    out = (o.view(B, H, 1, D), lse.view(B, H, 1))
    return out + ((m, d, op),) if return_partials else out
