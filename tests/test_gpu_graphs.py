"""The entry points under HIP graph capture, the use the allocation-free decode is for:
fa_forward, fa_backward, fa_decode_noalloc and the chained scan fa_softmax_scan_ws (its
workspace cleared by a kernel of its own) recorded into one graph (torch.cuda.graph
captures the stream the binding launches on), then replayed several times with new
inputs copied into the captured tensors and eager work of the same calls in between.

Every kernel here is deterministic (a fixed reduction order; the scan's blocks find their
predecessors' words long before their bound of polls runs out), so each replay must
reproduce the eager calls on the same inputs bit for bit; the eager calls
are themselves compared with the oracle by the parity tests. The library records no
memset and allocates nothing, so nothing else needs to stay out of the graph.
"""
import math

import pytest
import torch

from exact_io_aware_22_amd import fa
from exact_io_aware_22_amd.workloads import random_tensor

pytestmark = pytest.mark.gpu

B, H, N, D = 2, 4, 777, 128
L, SPLITS = 3001, 16
SCAN_N = 32768  # float32 rows of 128 KB: the chained scan (16 blocks per row)
SCALE = 1.0 / math.sqrt(D)


def say(msg):
    print(msg, flush=True)


def fresh_inputs(seed):
    shape = (B, H, N, D)
    return {
        "q": random_tensor(shape, seed, torch.bfloat16, sigma=2.0),
        "k": random_tensor(shape, seed + 1, torch.bfloat16, sigma=2.0),
        "v": random_tensor(shape, seed + 2, torch.bfloat16),
        "do": random_tensor(shape, seed + 3, torch.bfloat16),
        "q1": random_tensor((B, H, 1, D), seed + 4, torch.bfloat16),
        "kc": random_tensor((B, H, L, D), seed + 5, torch.bfloat16, sigma=2.0),
        "vc": random_tensor((B, H, L, D), seed + 6, torch.bfloat16),
        "rows": random_tensor((8, SCAN_N), seed + 7, torch.float32, sigma=8.0),
    }


def outputs():
    f32 = dict(dtype=torch.float32, device="cuda")
    return {
        "o": torch.full((B, H, N, D), float("nan"), **f32),
        "lse": torch.full((B, H, N), float("nan"), **f32),
        "delta": torch.full((B, H, N), float("nan"), **f32),
        "dq": torch.full((B, H, N, D), float("nan"), **f32),
        "dk": torch.full((B, H, N, D), float("nan"), **f32),
        "dv": torch.full((B, H, N, D), float("nan"), **f32),
        "od": torch.full((B * H, D), float("nan"), **f32),
        "lsed": torch.full((B * H,), float("nan"), **f32),
        "sm": torch.full((8, SCAN_N), float("nan"), **f32),
        "sd": torch.full((8, SCAN_N), float("nan"), **f32),
        # the chained scan's workspace (cleared by the call itself, so it is an output)
        "ws": torch.zeros(fa.fa_scan_workspace_bytes(8, SCAN_N), dtype=torch.uint8,
                          device="cuda"),
    }


def calls(x, y):
    """One training step's attention (forward, then backward from its o and lse), one
    decode step and one chained scan, all on the current stream."""
    fa.fa_forward(x["q"], x["k"], x["v"], y["o"], y["lse"], SCALE, True)
    fa.fa_backward(x["q"], x["k"], x["v"], y["o"], y["lse"], x["do"], y["delta"], y["dq"],
                   y["dk"], y["dv"], SCALE, True)
    fa.fa_decode_noalloc(x["q1"], x["kc"], x["vc"], y["od"], y["lsed"], SCALE, SPLITS)
    fa.fa_softmax_scan_ws(x["rows"], y["sm"], y["sd"], y["ws"])


def test_captured_calls_replay_like_eager_calls():
    assert torch.cuda.is_available(), "this test needs the GPU"
    fa.load()
    static_in = {name: t.cuda() for name, t in fresh_inputs(5000).items()}
    static_out = outputs()
    # an eager call first: the allocation-free decode looks up its scratch address on
    # its first call on a device, which must not happen during capture
    calls(static_in, static_out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(static_in, static_out)
    torch.cuda.synchronize()
    for replay in range(4):
        new = fresh_inputs(5100 + 10 * replay)
        for name, t in new.items():
            static_in[name].copy_(t.cuda())
        say(f"replay {replay}: B={B} H={H} N={N} D={D}, decode L={L} splits={SPLITS}")
        graph.replay()
        torch.cuda.synchronize()
        # the same calls eagerly, on copies of the inputs, into fresh outputs
        eager_in = {name: t.clone() for name, t in static_in.items()}
        eager_out = outputs()
        calls(eager_in, eager_out)
        torch.cuda.synchronize()
        for name in static_out:
            if name == "ws":
                continue  # scratch: its contents after a call mean nothing
            got, want = static_out[name], eager_out[name]
            assert bool(torch.isfinite(want).all()), f"replay {replay}: eager {name} not finite"
            assert torch.equal(got, want), (
                f"replay {replay}: {name} differs from the eager call "
                f"(max |diff| {float((got - want).abs().max()):.3e})")
