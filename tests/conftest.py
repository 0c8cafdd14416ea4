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
