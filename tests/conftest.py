import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def rel_err_ok(got, ref, tol):
    """Per-entry check |g - r| <= tol * max(|r|, rms(r)).  The rms floor keeps
    near-zero entries of random contractions from demanding a pure relative
    bound they cannot meet; a scalar uses |r| alone."""
    import numpy as np
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    if ref.size == 1:
        floor = np.abs(ref)
    else:
        floor = np.maximum(np.abs(ref), np.sqrt(np.mean(np.abs(ref) ** 2)))
    err = np.abs(got - ref)
    bad = err > tol * floor
    return (not bad.any()), float(np.max(err / np.where(floor > 0, floor, 1.0))) if ref.size else 0.0
