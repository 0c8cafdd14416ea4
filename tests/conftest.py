import contextlib
import json
import math
import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def exact(expr: str) -> float:
    """Evaluate a golden fixture's exact expression (numbers, + - * /, log, inf)."""
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "inf": math.inf}))


def load_golden(name: str) -> dict:
    return json.loads((GOLDEN / name).read_text())


def exact_array(rows):
    import numpy as np

    if rows and isinstance(rows[0], list):
        return np.array([[exact(x) for x in r] for r in rows], dtype=np.float64)
    return np.array([exact(x) for x in rows], dtype=np.float64)


# Threads for the oracle at full size: the host cores this process may run on, at most
# 16 (one GPU's share of a shared host); each worker's BLAS runs single-threaded.
ORACLE_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


@contextlib.contextmanager
def one_blas_thread():
    """BLAS pinned to one thread while the oracle's own workers run in parallel."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        yield
        return
    with threadpool_limits(limits=1):
        yield


def parallel_map(fn, items, workers=None):
    """fn over items on a thread pool (numpy and BLAS release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    items = list(items)
    workers = ORACLE_WORKERS if workers is None else workers
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
