"""Host checks of bench.py's contract that need no GPU: it measures one GPU only, so
--gpus above 1 (or a WORLD_SIZE above 1) exits with a message before touching torch's
device code, and the peaks it divides by are MI355X's published dense figures."""
import os
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def run_bench(*args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_exits_with_a_message():
    r = run_bench(env_extra={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_published_peaks():
    sys.path.insert(0, str(ROOT))
    import bench

    assert bench.PEAK_BF16_TFLOPS == 2500.0  # dense bf16 MFMA
    assert bench.PEAK_HBM_GBS == 8000.0      # HBM3E
    assert bench.HEADLINE == "large_score_causal_d128"


def test_stream_fraction_against_the_two_ceilings():
    sys.path.insert(0, str(ROOT))
    import bench

    # Units cancel, so plain numbers: ceilings 7 (read) and 5 (write) bytes per time
    # unit. A kernel reading 1 and writing 4 at exactly the ceilings takes 1/7 + 4/5;
    # its roofline over all 5 bytes then reports 5 / (1/7 + 4/5).
    t = 1 / 7 + 4 / 5
    assert abs(bench.stream_fraction(1, 4, 5, 5 / t, 7, 5) - 1.0) < 1e-12
    assert abs(bench.stream_fraction(1, 4, 5, 5 / (2 * t), 7, 5) - 0.5) < 1e-12  # twice as slow
    # A roofline that credits only the reads (as the decode's does): the writes still
    # take ceiling time.
    t = 1 / 7 + 0.01 / 5
    assert abs(bench.stream_fraction(1, 0.01, 1, 1 / t, 7, 5) - 1.0) < 1e-12


def test_median_and_min():
    sys.path.insert(0, str(ROOT))
    import bench

    assert bench.median_min([3.0, 1.0, 2.0]) == (2.0, 1.0)
    assert bench.median_min([4.0, 1.0, 3.0, 2.0]) == (2.5, 1.0)

