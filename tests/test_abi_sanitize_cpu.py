"""The C ABI's validation layer and the launchers' host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (tests/sanitize/abi_host_check.cpp).

Two programs are built in a temporary directory:
  - api.cpp with stub launchers (g++), checking that only validated arguments reach a
    launcher;
  - api.cpp with the real launchers, whose .hip sources are compiled for the host only
    (no device code) against stubs of the HIP runtime calls they make (clang++), checking
    every launch configuration they form.
Both sweep every entry point over extreme arguments; a sanitizer report fails the test.
No GPU is used and nothing is launched.
"""
import os
import re
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "exact_io_aware_22_amd" / "csrc"
CHECK = ROOT / "tests" / "sanitize" / "abi_host_check.cpp"
ROCM = Path(os.environ.get("ROCM_PATH", "/opt/rocm"))
HIPCC = ROCM / "bin" / "hipcc"
CLANGXX = ROCM / "llvm" / "bin" / "clang++"
INCLUDES = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM / 'include'}", f"-I{ROOT / 'include'}",
            f"-I{CSRC}"]
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ITERATIONS = "200000"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout}\n{res.stderr}"
    return res


def _check_output(res):
    text = res.stdout + res.stderr
    assert "runtime error" not in text and "ERROR: AddressSanitizer" not in text, text
    assert f"{ITERATIONS} sweep iterations, all checks passed" in res.stdout, text


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_validation_with_stub_launchers(tmp_path):
    exe = tmp_path / "abi_check"
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, *INCLUDES, str(CSRC / "api.cpp"), str(CHECK),
          "-o", str(exe)])
    _check_output(_run([str(exe), ITERATIONS], env=ENV, timeout=300))


@pytest.mark.skipif(not (HIPCC.exists() and CLANGXX.exists()), reason="ROCm toolchain missing")
def test_launcher_host_code_with_stub_runtime(tmp_path):
    objs = []
    hip_sources = sorted(CSRC.glob("*.hip"))
    assert hip_sources
    procs = []
    for src in hip_sources:  # host side only; sanitizers apply to the host pass
        obj = tmp_path / f"{src.stem}.o"
        cmd = [str(HIPCC), "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", *INCLUDES[1:], "-c", str(src),
               "-o", str(obj)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{out}\n{err}"
    for src, define in ((CSRC / "api.cpp", []), (CHECK, ["-DFA_WITH_LAUNCHERS"])):
        obj = tmp_path / f"{src.stem}.o"
        _run([str(CLANGXX), "-std=c++17", "-O1", "-g", *SAN, *define, *INCLUDES, "-c", str(src),
              "-o", str(obj)])
        objs.append(obj)
    # Each host object refers to its (absent) embedded device image; define empty ones.
    undefined = _run(["nm", "-u", *map(str, objs)]).stdout
    fatbins = sorted(set(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", undefined)))
    assert len(fatbins) == len(hip_sources), fatbins
    stub = tmp_path / "fatbins.cpp"
    stub.write_text("".join(f'extern "C" const char {n}[1] = {{0}};\n' for n in fatbins))
    _run([str(CLANGXX), "-c", str(stub), "-o", str(tmp_path / "fatbins.o")])
    exe = tmp_path / "abi_check_launchers"
    _run([str(CLANGXX), *SAN, *map(str, objs), str(tmp_path / "fatbins.o"), "-o", str(exe)])
    _check_output(_run([str(exe), ITERATIONS], env=ENV, timeout=300))
