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
