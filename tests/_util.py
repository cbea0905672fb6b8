"""Shared test helpers (tolerance metric, fixtures on disk)."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerances on max|x - ref| / rms(ref): bf16 operands with fp32 accumulation,
# and the all-fp32 path.
TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def rel_err(x, ref) -> float:
    """max |x - ref| / sqrt(mean(ref^2)), the tolerance metric used throughout."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    rms = float(np.sqrt(np.mean(ref * ref)))
    diff = float(np.max(np.abs(x - ref)))
    return diff / rms if rms > 0.0 else diff


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
