"""Checks on the gfx950 code the compiler generates for the two kernels that stage tiles
with direct global -> LDS loads (fwd_bf16.hip, bwd_bf16.hip).

Those loads are issued from inline assembly that sets M0 (the LDS destination) right
before each load. The compiler is not told about M0 (it treats it as reserved and does
not preserve it across inline assembly), so the code is correct only while the
compiler itself neither keeps a value in M0 across such a load nor uses an instruction
that reads M0 implicitly. This test compiles both sources with the library's flags and
checks exactly that, so a toolchain or source change that breaks the assumption fails
here, on the CPU, before any GPU run.
"""
import re
import subprocess

import pytest

from exact_io_aware_22_amd import build

# Instructions that read M0 without naming it as an operand.
IMPLICIT_M0 = re.compile(r"^\s*(s_sendmsg|s_sendmsghalt|s_movrel|v_movrel|ds_gws|v_interp|"
                         r"s_ttracedata|buffer_load\S*.*\blds\b|global_load_lds(?!_dwordx4))")


def device_asm(src: str) -> str:
    cmd = [build._hipcc(), *[f for f in build.HIP_FLAGS if f not in ("-fPIC", "-Wall")],
           "-x", "hip", f"-I{build.INCLUDE}", f"-I{build.CSRC}", "--cuda-device-only", "-S",
           str(build.CSRC / src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


@pytest.mark.parametrize("src", ["fwd_bf16.hip", "bwd_bf16.hip"])
def test_m0_is_only_the_staging_loads_destination(src):
    lines = [l.split(";")[0].strip() for l in device_asm(src).splitlines()]
    code = [l for l in lines if l and not l.startswith((".", "//")) and not l.endswith(":")]
    writes = loads = 0
    for i, l in enumerate(code):
        assert not IMPLICIT_M0.match(l), f"{src}: instruction that reads M0 implicitly: {l}"
        if re.search(r"\bm0\b", l):
            # the only M0 use: our own write, then the wait state, then the staging load
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"{src}: M0 used by the compiler: {l}"
            assert code[i + 1] == "s_nop 0" and code[i + 2].startswith("global_load_lds_dwordx4"), \
                f"{src}: M0 write not followed by its load: {code[i:i + 3]}"
            writes += 1
        if l.startswith("global_load_lds_dwordx4"):
            loads += 1
    assert writes > 0 and writes == loads, (writes, loads)


def kernel_resources(asm: str):
    """(name, vgprs, agprs, scratch bytes per lane, LDS bytes) of every kernel, from the
    code object metadata the compiler emits with the assembly."""
    out = []
    for block in re.split(r"\n\s*- \.", asm.split("amdhsa.kernels:")[-1])[1:]:
        def field(key):
            m = re.search(rf"\.?{key}:\s+(\S+)", block)
            return m.group(1) if m else None
        name = field("name")
        if name is None or field("vgpr_count") is None:
            continue
        out.append((name, int(field("vgpr_count")), int(field("agpr_count") or 0),
                    int(field("private_segment_fixed_size")),
                    int(field("group_segment_fixed_size"))))
    return out


@pytest.mark.parametrize("src,kernels", [
    ("fwd_bf16.hip", ["fwd_bf16_kernel"]),
    ("bwd_bf16.hip", ["dq_kernel", "dkdv_kernel"]),
    ("decode.hip", ["decode_partials_kernel", "decode_partials_wave_kernel", "combine_kernel"]),
    ("reduce.hip", ["row_reduce_kernel", "row_scan_kernel"]),
])
def test_hot_kernels_keep_their_occupancy_without_scratch(src, kernels):
    """Every instance of the hot kernels compiles without scratch (no spilled registers,
    no private arrays) and within 256 VGPRs, so two wavefronts fit each SIMD; the
    MFMA kernels use 160 KB of LDS or less, one workgroup per CU."""
    res = kernel_resources(device_asm(src))
    for k in kernels:
        mine = [r for r in res if k + "I" in r[0]]
        assert mine, f"{src}: no instance of {k} in {[r[0] for r in res]}"
        for name, vgpr, agpr, scratch, lds in mine:
            assert scratch == 0, f"{name}: {scratch} bytes of scratch per lane"
            assert vgpr + agpr <= 256, f"{name}: {vgpr} VGPRs + {agpr} AGPRs"
            assert lds <= 160 * 1024, f"{name}: {lds} bytes of LDS"
