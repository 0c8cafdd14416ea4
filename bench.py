#!/usr/bin/env python3
"""Benchmark of the exact attention forward and split-KV decode on one MI355X.

Prints ONE JSON line. A step is one fa_forward over the headline workload
(bf16, B=2, H=32, N=8192, D=128, causal, q and k ~ N(0, 9)); `value` is its
throughput in TFLOP/s under the 4*B*H*N^2*D (halved for causal) convention.
The same line carries the backward pass on the headline inputs (TFLOP/s, 2.5x-forward
convention), the split-KV decode (bf16, B=16, H=32, one query row, 32768
keys, D=128, 64 chunks of 512) as HBM GB/s, the other prefill workloads' rates,
a live roofline of the dominant kernel, and the fp64 oracle timed on the host cores
(its only use here: parity at these sizes is checked by the GPU tests).

Timing: inputs are resident in HBM before the timed region; at least W untimed
warm-up steps and at least 0.25 s of them, then K steps bracketed by torch.cuda.synchronize() and HIP events recorded
on the stream the kernels are launched on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
HEADLINE = "large_score_causal_d128"
DECODE = "split_kv_decode"
MASKED = ["sliding_window_4096_causal_d128", "sliding_window_1024_causal_d128",
          "varlen_causal_d128"]
EXTRA = ["batched_prefill_d64", "batched_prefill_d64_causal", "long_context_causal_32768",
         "long_context_causal_32767", "single_head_fp32"]
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector ALU
KERNEL_SOURCES = {
    "fwd_bf16_kernel": "exact_io_aware_22_amd/csrc/fwd_bf16.hip",
    "decode_partials_kernel": "exact_io_aware_22_amd/csrc/decode.hip",
    "row_reduce_kernel<SoftmaxMonoid>": "exact_io_aware_22_amd/csrc/reduce.hip",
    "row_reduce_kernel<WelfordMonoid>": "exact_io_aware_22_amd/csrc/reduce.hip",
    "row_scan_kernel<SoftmaxMonoid>": "exact_io_aware_22_amd/csrc/reduce.hip",
    "row_scan_kernel<WelfordMonoid>": "exact_io_aware_22_amd/csrc/reduce.hip",
    "dq_kernel + dkdv_kernel": "exact_io_aware_22_amd/csrc/bwd_bf16.hip",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(rel: str) -> str:
    return hashlib.sha256((ROOT / rel).read_bytes()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were
    taken on the current kernel source (else None)."""
    f = ROOT / "profiles" / "pmc_traffic.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get(kernel, {}).get(workload)
    except (ValueError, AttributeError):
        return None
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


CPU_SHARE = 16  # host cores one GPU's jobs may use on a shared host
WARM_SECONDS = 0.25  # the clock ramps up over the first tens of milliseconds of load


def time_launches(fn, steps: int, warmup: int, torch):
    """Average milliseconds per call of fn(), HIP events on the current stream.

    Warm-up runs at least `warmup` calls and at least WARM_SECONDS of them, so a short
    kernel measured after an idle stretch is not timed on a cold clock."""
    t_end = time.perf_counter() + WARM_SECONDS
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def stream_fraction(read_bytes: float, write_bytes: float, alg_bytes: float, achieved_gbs: float,
                    read_gbs: float, write_gbs: float) -> float:
    """Fraction of the measured HBM ceiling for a kernel that reads read_bytes and writes
    write_bytes per launch and whose roofline reports achieved_gbs over alg_bytes: the
    time a read stream and a write stream of those bytes take (at read_gbs, write_gbs),
    over the kernel's measured time (alg_bytes / achieved_gbs)."""
    t_ceiling = read_bytes / read_gbs + write_bytes / write_gbs
    t_measured = alg_bytes / achieved_gbs
    return t_ceiling / t_measured


def median_min(times_ms):
    """Median (mean of the middle two for an even count) and minimum of per-call times."""
    t = sorted(times_ms)
    mid = len(t) // 2
    return (t[mid] if len(t) % 2 else 0.5 * (t[mid - 1] + t[mid])), t[0]


def time_each(fn, calls: int, torch):
    """Per-call milliseconds, HIP events around each call on the current stream: the
    median and the minimum over `calls` launches (run after time_launches, so warm)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    median, fastest = median_min([a.elapsed_time(b) for a, b in ev])
    return {"calls": calls, "median_ms": median, "min_ms": fastest}


def measured_ceilings(steps: int, warmup: int, torch, fa):
    """The chip's sustained rates, the denominators of the fractions of measured (not
    published) peaks: the library's MFMA-only loop (random bf16 register operands, two
    wavefronts per SIMD), its read-only and write-only streams (16-byte non-temporal loads
    and stores of 2 GiB), and its copy from one read into two write streams at the prefix
    scans' byte ratios.
    A bf16 GEMM (torch.mm) and a device copy are reported beside them as library
    references."""
    blocks, iters = 1024, 256
    chk = torch.empty(blocks * 512, device="cuda")
    ms_mfma = time_launches(lambda: fa.fa_calibrate_mfma(chk, blocks, iters, seed=1), steps,
                            warmup, torch)
    mfma_flops = 2 ** 19 * 8 * blocks * iters
    nbytes = 2 << 30
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    # the streams' best grid: the best of a small sweep (one contiguous span per workgroup)
    ms_read, ms_write = [], []
    for rblocks in (512, 1024):
        fold = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
        ms_read.append(time_launches(lambda: fa.fa_calibrate_read(x, fold, rblocks), steps,
                                     warmup, torch))
        ms_write.append(time_launches(lambda: fa.fa_calibrate_write(x, 7, rblocks), steps,
                                      warmup, torch))
        del fold
    ms_read, ms_write = min(ms_read), min(ms_write)
    del chk, x
    # one read and two write streams at the prefix scans' byte ratios (each output 1x the
    # input for float32 input, 2x for bfloat16), no arithmetic: 1 GiB read
    mbytes = 1 << 30
    mx = torch.ones(mbytes // 4, dtype=torch.int32, device="cuda")
    mix = {}
    for ratio in (1, 2):
        my = torch.empty(2 * ratio * mbytes // 4, dtype=torch.int32, device="cuda")
        ms_mix = min(time_launches(lambda: fa.fa_calibrate_mix(mx, my, ratio, mblocks), steps,
                                   warmup, torch) for mblocks in (8192, 16384, 32768))
        mix[str(ratio)] = (1 + 2 * ratio) * mbytes / (ms_mix * 1e-3) / 1e9
        del my
    del mx
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ms_mm = time_launches(lambda: torch.mm(a, b, out=c), steps, warmup, torch)
    del a, b, c
    y = torch.empty_like(x)
    ms_cp = time_launches(lambda: y.copy_(x), steps, warmup, torch)
    del x, y
    torch.cuda.empty_cache()
    return {
        "mfma_bf16_tflops": mfma_flops / (ms_mfma * 1e-3) / 1e12,
        "mfma_bf16": f"fa_calibrate_mfma: {blocks} workgroups x 8 wavefronts x {iters} rounds "
                     "of 16 32x32x16 bf16 products, random operands",
        "read_gbs": nbytes / (ms_read * 1e-3) / 1e9,
        "read": f"fa_calibrate_read: {nbytes >> 30} GiB, 16-byte non-temporal loads, best of "
                "512 and 1024 workgroups",
        "write_gbs": nbytes / (ms_write * 1e-3) / 1e9,
        "write": f"fa_calibrate_write: {nbytes >> 30} GiB, 16-byte non-temporal stores, best of "
                 "512 and 1024 workgroups",
        "mix_gbs": mix,
        "mix": "fa_calibrate_mix: 1 GiB read, written to two streams of ratio x 1 GiB (keys: "
               "ratio), bytes read + written per second, best of 8192, 16384 and 32768 workgroups",
        "library_reference": {
            "bf16_gemm_tflops": 2 * n ** 3 / (ms_mm * 1e-3) / 1e12,
            "bf16_gemm": f"torch.mm {n}x{n}x{n}, N(0, 1) operands",
            "copy_gbs": 2 * nbytes / (ms_cp * 1e-3) / 1e9,
            "copy": f"device copy of {nbytes >> 30} GiB, bytes read + written"},
    }


def bench_prefill(name: str, steps: int, warmup: int, torch, fa, make_inputs, W,
                  per_launch=False, graph=False):
    w = W[name]
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty(w.B, w.H, w.N, w.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    launch = lambda: fa.fa_forward(qd, kd, vd, o, lse, w.scale, w.causal)  # noqa: E731
    ms = time_launches(launch, steps, warmup, torch)
    res = {"workload": name, "ms": ms, "tflops": w.flops() / (ms * 1e-3) / 1e12}
    if per_launch:
        res["per_launch"] = time_each(launch, max(20, steps), torch)
    if graph:
        # A launch shorter than the binding's host-side cost is timed back to back from a
        # HIP graph of `reps` launches, so the GPU never waits for the host between them.
        reps = 64
        launch()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                launch()
        ms_graph = time_launches(g.replay, max(10, steps // 4), 3, torch) / reps
        res["graph"] = {"launches_per_replay": reps, "ms": ms_graph,
                        "tflops": w.flops() / (ms_graph * 1e-3) / 1e12}
        del g
    del qd, kd, vd, o, lse
    return res, (q, k, v)


def bench_decode(steps: int, warmup: int, torch, fa, make_inputs, W):
    w = W[DECODE]
    log(f"drawing {DECODE} inputs")
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    BH, S, D = w.B * w.H, w.splits, w.D
    m = torch.empty(BH, S, device="cuda")
    d = torch.empty(BH, S, device="cuda")
    op = torch.empty(BH, S, D, device="cuda")
    o = torch.empty(BH, D, device="cuda")
    lse = torch.empty(BH, device="cuda")

    def partials():
        fa.fa_decode_partials(qd, kd, vd, m, d, op, w.scale, S)

    def combine():
        fa.fa_combine_partials(m, d, op, o, lse)

    def step():
        partials()
        combine()

    ms_step = time_launches(step, steps, warmup, torch)
    ms_part = time_launches(partials, steps, warmup, torch)
    ms_comb = time_launches(combine, steps, warmup, torch)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    ms_noalloc = time_launches(lambda: fa.fa_decode_noalloc(qd, kd, vd, o2, lse2, w.scale, S),
                               steps, warmup, torch)
    esz = 2
    kv_bytes = 2 * w.B * w.H * w.L * w.D * esz
    q_bytes = w.B * w.H * w.D * esz
    out_bytes = BH * D * 4 + BH * 4
    step_bytes = kv_bytes + q_bytes + out_bytes
    part_bytes = kv_bytes + q_bytes
    achieved = part_bytes / (ms_part * 1e-3) / 1e9
    traffic = measured_traffic("decode_partials_kernel", DECODE)
    res = {
        "workload": DECODE, "value": step_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
        "ms_per_step": ms_step, "ms_partials": ms_part, "ms_combine": ms_comb,
        "ms_noalloc": ms_noalloc, "noalloc_gbs": step_bytes / (ms_noalloc * 1e-3) / 1e9,
        "bytes_per_step": step_bytes,
        "config": {"B": w.B, "H": w.H, "L": w.L, "D": w.D, "splits": S, "dtype": "bf16"},
        "roofline": {"kernel": "decode_partials_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": part_bytes,
                     "read_bytes": part_bytes, "write_bytes": BH * S * (D + 2) * 4},
    }
    del qd, kd, vd, o2, lse2
    torch.cuda.empty_cache()
    res["one_gpu_share"] = bench_decode_share(steps, warmup, torch, fa, q, k, v, w)
    return res


def bench_decode_share(steps: int, warmup: int, torch, fa, q, k, v, w, shards: int = 8):
    """What one GPU of an 8-GPU split-KV decode does: fa_decode_partials over its share of
    the keys (L / 8 = 4096 per head, B=16, H=32) in 8 and in 64 chunks, and the merge of
    all 8 shards' 64 partials each (rows = 512, 512 partials per row) by one
    fa_combine_partials call, as after an all-gather of the partials."""
    per = w.L // shards
    qd = q.cuda()
    ks = k[:, :, :per].contiguous().cuda()
    vs = v[:, :, :per].contiguous().cuda()
    BH, D = w.B * w.H, w.D
    out = {"keys_per_head": per, "shards": shards, "partials": []}
    kv_bytes = 2 * BH * per * D * 2 + BH * D * 2
    for splits in (8, 64):
        m = torch.empty(BH, splits, device="cuda")
        d = torch.empty(BH, splits, device="cuda")
        op = torch.empty(BH, splits, D, device="cuda")
        ms = time_launches(lambda: fa.fa_decode_partials(qd, ks, vs, m, d, op, w.scale, splits),
                           steps, warmup, torch)
        gbs = kv_bytes / (ms * 1e-3) / 1e9
        out["partials"].append({"splits": splits, "ms": ms, "gbs": gbs,
                                "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
                                "algorithmic_bytes": kv_bytes})
        del m, d, op
    P = shards * w.splits
    m = torch.empty(BH, P, device="cuda")
    d = torch.empty(BH, P, device="cuda")
    op = torch.empty(BH, P, D, device="cuda")
    for s in range(shards):  # each shard's partials, as its GPU would have produced them
        ksl = k[:, :, s * per:(s + 1) * per].contiguous().cuda()
        vsl = v[:, :, s * per:(s + 1) * per].contiguous().cuda()
        mp, dp = torch.empty(BH, w.splits, device="cuda"), torch.empty(BH, w.splits, device="cuda")
        opp = torch.empty(BH, w.splits, D, device="cuda")
        fa.fa_decode_partials(qd, ksl, vsl, mp, dp, opp, w.scale, w.splits)
        m.view(BH, shards, w.splits)[:, s] = mp
        d.view(BH, shards, w.splits)[:, s] = dp
        op.view(BH, shards, w.splits, D)[:, s] = opp
        del ksl, vsl, mp, dp, opp
    o = torch.empty(BH, D, device="cuda")
    lse = torch.empty(BH, device="cuda")
    ms = time_launches(lambda: fa.fa_combine_partials(m, d, op, o, lse), steps, warmup, torch)
    comb_bytes = BH * P * (D + 2) * 4 + BH * (D + 1) * 4
    out["combine_remote"] = {"rows": BH, "partials_per_row": P, "ms": ms,
                             "gbs": comb_bytes / (ms * 1e-3) / 1e9,
                             "algorithmic_bytes": comb_bytes}
    del qd, ks, vs, m, d, op, o, lse
    torch.cuda.empty_cache()
    return out


def measure_overlap(torch, fa, blocks: int = 256, iters: int = 4096):
    """fa_calibrate_overlap: milliseconds of each mode (one workgroup of 8 wavefronts per
    CU) and the share of the shorter role's time that runs concurrently with the other
    when one matrix and one vector wavefront share each SIMD:
    (t_matrix + t_vector - t_both) / min(t_matrix, t_vector); 1 = full overlap, 0 = none."""
    out_buf = torch.empty(blocks * 512, device="cuda")
    fa.fa_calibrate_overlap(out_buf, blocks, 0, 6)
    torch.cuda.synchronize()
    simd = out_buf.view(blocks, 8, 64)[:, :, 0].cpu()
    paired = bool(torch.equal(simd[:, :4], simd[:, 4:]))
    names = ["matrix_1_per_simd", "vector_1_per_simd", "matrix_and_vector_per_simd",
             "both_roles_every_wave", "matrix_2_per_simd", "vector_2_per_simd"]
    ms = {}
    for mode, name in enumerate(names):
        ms[name] = time_launches(lambda: fa.fa_calibrate_overlap(out_buf, blocks, iters, mode),
                                 5, 3, torch)
    t0, t1, t2 = ms[names[0]], ms[names[1]], ms[names[2]]
    clock = {}
    for mode, name in enumerate(names):  # the shader clock each mode ran at
        out_buf.zero_()
        fa.fa_calibrate_overlap(out_buf, blocks, iters, 8 + mode)
        torch.cuda.synchronize()
        t = out_buf.view(blocks, 8, 64).cpu()
        cyc, ticks = t[:, :, 0].flatten(), t[:, :, 32].flatten()
        live = ticks > 0
        clock[name] = float((cyc[live] / ticks[live]).median()) * 100.0  # MHz
    return {"blocks": blocks, "iters": iters, "ms": ms, "clock_mhz": clock,
            "waves_w_and_w_plus_4_share_a_simd": paired,
            "overlap_fraction": (t0 + t1 - t2) / min(t0, t1),
            "matrix_tflops_1_per_simd": 2 ** 15 * 16 * 4 * blocks * iters / (t0 * 1e-3) / 1e12}


def cpu_baseline(q, k, v, w, budget_s: float):
    """The fp64 oracle, as it is, on whole heads of the headline workload."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    host_cpus = len(os.sched_getaffinity(0))
    # The host is shared by the GPUs of its node and one GPU's jobs get 16 of its cores,
    # so the oracle takes every core this process may use, up to that share.
    cores = max(1, min(CPU_SHARE, host_cpus))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    heads, t_used = 0, 0.0
    try:
        if ctx:
            ctx.__enter__()
        t0 = time.perf_counter()
        for b in range(w.B):
            for h in range(w.H):
                oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                 w.scale, w.causal, row_block=512, workers=cores)
                heads += 1
                t_used = time.perf_counter() - t0
                if t_used >= budget_s:
                    break
            if t_used >= budget_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    flops = w.flops() / (w.B * w.H) * heads
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of {w.name} (all {w.N} rows each), fp64 numpy, "
                      f"BLAS 1 thread per worker",
            "seconds": t_used, "host_cpus_visible": host_cpus, "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: its model-name line, with the vendor,
    family, model and stepping fields (a virtualised host may give a short name)."""
    fields = {}
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if ":" not in line:
                if fields:
                    break  # the first processor's block is enough
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            if key in ("model name", "vendor_id", "cpu family", "model", "stepping"):
                fields.setdefault(key, val)
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    extra = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping")
                      if k in fields)
    return f"{name} ({extra})" if extra else name


def bench_backward(steps: int, warmup: int, torch, fa, make_inputs, W):
    """fa_backward (the dQ kernel, which also forms Delta, then the dK/dV kernel) on the
    headline workload's inputs with a seeded upstream gradient; flops under the usual
    2.5x-forward convention (five products: S recomputed, dV, dP, dQ, dK), halved for
    causal."""
    from exact_io_aware_22_amd.workloads import random_tensor

    w = W[HEADLINE]
    q, k, v = make_inputs(w)
    do = random_tensor(tuple(q.shape), 99, torch.bfloat16)
    qd, kd, vd, dd = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, w.scale, w.causal)
    delta = torch.empty(w.B, w.H, w.N, device="cuda")
    dq, dk, dv = (torch.empty(w.B, w.H, w.N, w.D, device="cuda") for _ in range(3))
    ms = time_launches(lambda: fa.fa_backward(qd, kd, vd, o, lse, dd, delta, dq, dk, dv, w.scale,
                                              w.causal), steps, warmup, torch)
    flops = 2.5 * w.flops()
    achieved = flops / (ms * 1e-3) / 1e12
    res = {"workload": HEADLINE, "ms_per_step": ms, "value": achieved, "unit": "TFLOP/s",
           "flop_convention": "2.5 x forward (5 products), halved for causal",
           "roofline": {"kernels": "dq_kernel + dkdv_kernel", "bound": "mfma",
                        "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / PEAK_BF16_TFLOPS,
                        "traffic": measured_traffic("dq_kernel + dkdv_kernel",
                                                    HEADLINE),
                        "algorithmic_flops_per_launch": flops}}
    del qd, kd, vd, dd, o, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def bench_masks(steps: int, warmup: int, torch, fa, W):
    """fa_forward_ext on the sliding-window and packed workloads; flops count the
    visible (query, key) pairs only (4*D per pair), so a window that skips tiles is
    not credited for work it does not do."""
    from exact_io_aware_22_amd.workloads import make_inputs, packed_inputs

    res = []
    for name in MASKED:
        w = W[name]
        log(f"timing {name}")
        if w.seqlens:
            q, k, v, cu = packed_inputs(w)
            cud = cu.cuda()
            max_len = max(w.seqlens)
        else:
            q, k, v = make_inputs(w)
            cu, cud, max_len = None, None, 0
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: fa.fa_forward_ext(qd, kd, vd, o, lse, w.scale, w.causal,
                                                     w.window_left, w.window_right, cud,
                                                     max_len), steps, warmup, torch)
        flops = w.flops()
        r = {"workload": name, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
             "visible_pairs": w.visible_pairs(), "algorithmic_flops_per_launch": flops}
        r["frac_of_bf16_peak"] = r["tflops"] / PEAK_BF16_TFLOPS
        res.append(r)
        del qd, kd, vd, o, lse, cud, cu
        torch.cuda.empty_cache()
    return res


def bench_reductions(steps: int, warmup: int, torch, fa):
    """fa_softmax_stats and fa_moments on their 1 GiB workloads, then the inclusive scans
    (fa_softmax_scan, fa_moments_scan) of the same rows: HBM-bound, so GB/s of
    algorithmic bytes (every element read once; two float32 outputs per row, or per
    element for a scan, written) against 8 TB/s."""
    from exact_io_aware_22_amd.workloads import ROW_WORKLOADS, make_rows

    res = []
    for name in sorted(ROW_WORKLOADS):
        w = ROW_WORKLOADS[name]
        log(f"timing {name}")
        x = make_rows(w)
        xd = x.cuda()
        a = torch.empty(w.rows, device="cuda")
        b = torch.empty(w.rows, device="cuda")
        softmax = name.startswith("softmax")
        fn = fa.fa_softmax_stats if softmax else fa.fa_moments
        ms = time_launches(lambda: fn(xd, a, b), steps, warmup, torch)
        nbytes = w.bytes_read() + w.bytes_written()
        gbs = nbytes / (ms * 1e-3) / 1e9
        kernel = "row_reduce_kernel<" + ("SoftmaxMonoid" if softmax else "WelfordMonoid") + ">"
        r = {"workload": name, "rows": w.rows, "n": w.n, "dtype": str(w.dtype).split(".")[-1],
             "ms": ms, "value": gbs, "unit": "GB/s",
             "roofline": {"kernel": kernel, "bound": "hbm", "achieved": gbs,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                          "traffic": measured_traffic(kernel, name),
                          "algorithmic_bytes_per_launch": nbytes,
                          "read_bytes": w.bytes_read(), "write_bytes": w.bytes_written()}}
        res.append(r)
        del a, b
        # the inclusive scan of the same rows: every position's state written (two
        # float32 outputs per element)
        sa = torch.empty(w.rows, w.n, device="cuda")
        sb = torch.empty(w.rows, w.n, device="cuda")
        # through the workspace entry point: rows of 2 to 64 whole 2048-element blocks
        # are shared by several workgroups (the clearing of the workspace included)
        ws = torch.empty(max(fa.fa_scan_workspace_bytes(w.rows, w.n, xd.dtype), 8), dtype=torch.uint8,
                         device="cuda")
        sfn = fa.fa_softmax_scan_ws if softmax else fa.fa_moments_scan_ws
        ms = time_launches(lambda: sfn(xd, sa, sb, ws), max(3, steps // 2), max(2, warmup // 2),
                           torch)
        rfn = fa.fa_softmax_scan if softmax else fa.fa_moments_scan
        ms_row = time_launches(lambda: rfn(xd, sa, sb), max(3, steps // 2), max(2, warmup // 2),
                               torch)
        nbytes = w.bytes_read() + 2 * 4 * w.rows * w.n
        gbs = nbytes / (ms * 1e-3) / 1e9
        skernel = "row_scan_kernel<" + ("SoftmaxMonoid" if softmax else "WelfordMonoid") + ">"
        rs = {"workload": name, "op": "inclusive scan", "ms": ms, "value": gbs, "unit": "GB/s",
              "workspace_bytes": int(fa.fa_scan_workspace_bytes(w.rows, w.n, xd.dtype)),
              "one_workgroup_per_row": {"ms": ms_row, "gbs": nbytes / (ms_row * 1e-3) / 1e9},
              "roofline": {"kernel": skernel, "bound": "hbm", "achieved": gbs,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                           "traffic": measured_traffic(skernel, name),
                           "algorithmic_bytes_per_launch": nbytes,
                           "read_bytes": w.bytes_read(), "write_bytes": 2 * 4 * w.rows * w.n}}
        res.append(rs)
        del x, xd, sa, sb, ws
        torch.cuda.empty_cache()
    return res


def copy_calibration(torch, nbytes: int, steps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": steps}))


def sustain(seconds: float, torch, fa, make_inputs, W):
    """Each kernel family launched back to back for `seconds` of wall time (after an idle
    stretch of the same length), one JSON line per phase with its start and end times
    (Unix seconds) and call count, for reading the board's power and clock sensors
    (amd-smi, sampled by the caller) against the phases. Prints as it goes."""
    def phase(name, fn):
        t0 = time.time()
        n = 0
        while time.time() < t0 + seconds:
            for _ in range(16):
                fn()
            torch.cuda.synchronize()
            n += 16
        print(json.dumps({"phase": name, "start": t0, "end": time.time(), "calls": n}), flush=True)

    t0 = time.time()
    time.sleep(seconds)
    print(json.dumps({"phase": "idle", "start": t0, "end": time.time(), "calls": 0}), flush=True)
    chk = torch.empty(1024 * 512, device="cuda")
    phase("mfma_only_loop", lambda: fa.fa_calibrate_mfma(chk, 1024, 256, seed=1))
    w = W[HEADLINE]
    q, k, v = (t.cuda() for t in make_inputs(w))
    o = torch.empty(w.B, w.H, w.N, w.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    phase("forward_" + HEADLINE, lambda: fa.fa_forward(q, k, v, o, lse, w.scale, w.causal))
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 100)
    do = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    delta = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    grads = [torch.empty_like(o) for _ in range(3)]
    phase("backward_" + HEADLINE,
          lambda: fa.fa_backward(q, k, v, o, lse, do, delta, *grads, w.scale, w.causal))
    del q, k, v, o, lse, do, delta, grads
    torch.cuda.empty_cache()
    wd = W[DECODE]
    qd, kd, vd = (t.cuda() for t in make_inputs(wd))
    od = torch.empty(wd.B * wd.H, wd.D, device="cuda")
    ld = torch.empty(wd.B * wd.H, device="cuda")
    phase("decode_" + DECODE, lambda: fa.fa_decode_noalloc(qd, kd, vd, od, ld, wd.scale, wd.splits))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward", "masks",
                                       "reductions", "copy", "ceilings", "overlap", "sustain"],
                    default="all")
    ap.add_argument("--workload", default=HEADLINE, choices=[HEADLINE] + EXTRA,
                    help="with --only prefill: the prefill workload to time (default: the "
                         "headline); its line then carries that workload's rate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--seconds", type=float, default=10.0,
                    help="with --only sustain: wall time of each phase")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path to time "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import torch

    from exact_io_aware_22_amd import fa
    from exact_io_aware_22_amd.workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        return 1
    fa.load()
    torch.cuda.set_device(0)

    if args.only == "copy":
        copy_calibration(torch, 1 << 30, args.steps)
        return 0
    if args.only == "ceilings":
        print(json.dumps({"ceilings": measured_ceilings(args.steps, args.warmup, torch, fa),
                          "overlap": measure_overlap(torch, fa)}))
        return 0
    if args.only == "overlap":
        print(json.dumps({"overlap": measure_overlap(torch, fa)}))
        return 0
    if args.only == "sustain":
        sustain(args.seconds, torch, fa, make_inputs, WORKLOADS)
        return 0

    out = {"metric": METRIC}
    if args.only != "prefill" and args.workload != HEADLINE:
        print("--workload applies to --only prefill", file=sys.stderr)
        return 2
    if args.only in ("all", "prefill"):
        name = args.workload
        w = WORKLOADS[name]
        log(f"timing {name}")
        head, (q, k, v) = bench_prefill(name, args.steps, args.warmup, torch, fa, make_inputs,
                                        WORKLOADS, per_launch=True,
                                        graph=w.dtype == torch.float32)
        # the float32 workload's launches are shorter than an eager call's host-side cost
        ms = head["graph"]["ms"] if "graph" in head else head["ms"]
        flops = w.flops()
        achieved = flops / (ms * 1e-3) / 1e12
        fp32 = w.dtype == torch.float32  # only when asked for with --workload
        peak = PEAK_FP32_VECTOR_TFLOPS if fp32 else PEAK_BF16_TFLOPS
        out.update({
            "value": achieved, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32" if fp32 else "bf16", "data": "synthetic",
            "config": {"workload": name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                       "causal": w.causal, "sigma_qk": w.sigma_qk, "parallelism": "single GPU"},
            "roofline": {"kernel": "fwd_f32_kernel" if fp32 else "fwd_bf16_kernel",
                         "bound": "alu" if fp32 else "mfma", "achieved": achieved,
                         "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                         "traffic": None if fp32 else measured_traffic("fwd_bf16_kernel", name),
                         "algorithmic_flops_per_launch": flops},
        })
        out["per_launch"] = head["per_launch"]
        if "graph" in head:
            out["graph"] = head["graph"]
        if args.only == "all" and not args.no_cpu_baseline:
            log("timing the fp64 oracle on host cores")
            out["cpu_baseline"] = cpu_baseline(q, k, v, w, args.cpu_seconds)
        del q, k, v
        if args.only == "all" and not args.no_extra:
            out["also"] = []
            for name in EXTRA:
                log(f"timing {name}")
                fp32 = WORKLOADS[name].dtype == torch.float32
                r, _ = bench_prefill(name, max(3, args.steps // 2), max(1, args.warmup // 2), torch,
                                     fa, make_inputs, WORKLOADS, per_launch=fp32, graph=fp32)
                if fp32:
                    # float32 inputs take the vector-ALU kernels; at this size one launch is
                    # a few microseconds, so its time, not a fraction, is the figure: the
                    # kernel's from graph replay, and one eager call's through the binding
                    r["us"] = r["graph"]["ms"] * 1e3
                    r["us_eager_call"] = r["ms"] * 1e3
                    r["frac_of_fp32_vector_peak"] = r["graph"]["tflops"] / PEAK_FP32_VECTOR_TFLOPS
                else:
                    r["frac_of_bf16_peak"] = r["tflops"] / PEAK_BF16_TFLOPS
                out["also"].append(r)
                torch.cuda.empty_cache()
    if args.only in ("all", "backward"):
        log(f"timing the backward on {HEADLINE}")
        out["backward"] = bench_backward(max(3, args.steps // 5), max(2, args.warmup // 10), torch,
                                         fa, make_inputs, WORKLOADS)
    if args.only in ("all", "masks"):
        out["masks"] = bench_masks(max(3, args.steps // 2), max(2, args.warmup // 4), torch, fa,
                                   WORKLOADS)
    if args.only in ("all", "reductions"):
        out["reductions"] = bench_reductions(args.steps, args.warmup, torch, fa)
    if args.only in ("all", "decode"):
        log(f"timing {DECODE}")
        out["decode"] = bench_decode(args.steps, args.warmup, torch, fa, make_inputs, WORKLOADS)
        if args.only == "decode":
            dec = out["decode"]
            out.update({"value": dec["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                        "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
                        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                        "dtype": "bf16", "data": "synthetic",
                        "config": {"workload": DECODE, "parallelism": "single GPU"},
                        "roofline": dec["roofline"]})
    if args.only == "all":
        # Measured last, so the headline is not timed on a clock the GEMM has heated.
        log("timing the measured ceilings (MFMA-only loop, read and write streams, library references)")
        ceil = measured_ceilings(10, 5, torch, fa)
        ceil["overlap"] = measure_overlap(torch, fa)
        out["ceilings"] = ceil
        mfma_rooflines = [out.get("roofline"), out.get("backward", {}).get("roofline")]
        for r in mfma_rooflines:
            if r:
                r["frac_of_measured"] = r["achieved"] / ceil["mfma_bf16_tflops"]
        hbm_rooflines = [out.get("decode", {}).get("roofline")]
        hbm_rooflines += [r.get("roofline") for r in out.get("reductions", [])]
        for r in hbm_rooflines:
            if r:
                r["frac_of_measured"] = stream_fraction(
                    r["read_bytes"], r["write_bytes"], r["algorithmic_bytes_per_launch"],
                    r["achieved"], ceil["read_gbs"], ceil["write_gbs"])
                # a scan reads one stream and writes two: against a plain copy with the
                # same mix (reads and writes at once cost more than either stream alone)
                ratio = str(round(r["write_bytes"] / (2 * r["read_bytes"])))
                if r.get("kernel", "").startswith("row_scan_kernel") and ratio in ceil["mix_gbs"]:
                    r["frac_of_same_mix_copy"] = r["achieved"] / ceil["mix_gbs"][ratio]
    out["host"] = platform.node()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
