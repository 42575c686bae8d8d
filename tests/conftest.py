import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full workload sizes)")


def rel_errors(x, y):
    """Tensor-level relative errors of x against the reference y:
    max|x-y| / max|y| and mean|x-y| / mean|y| (element-wise relative error is
    ill-posed near zero)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.abs(x - y)
    return float(d.max() / np.abs(y).max()), float(d.mean() / np.abs(y).mean())


@pytest.fixture
def rel():
    return rel_errors
