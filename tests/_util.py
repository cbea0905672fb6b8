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


# bf16 round-to-nearest-even moves a value by at most 2^-8 of its magnitude
# (half an ulp with 8 significant bits).  A bf16 *output* therefore cannot be
# closer to the exact result than that, whatever the arithmetic before the
# store: a perfect fp64 result rounded to bf16 already exceeds 2e-2 * rms on
# heavy-tailed outputs.  Outputs stored in bf16 are checked elementwise as
#     |x - ref| <= tol * rms(ref) + 2^-8 * |ref|
# i.e. the stated bound on the arithmetic plus the storage rounding of the
# output itself.  fp32 outputs (states, the fp32 path) use the bound alone.
BF16_STORE = 2.0 ** -8


def bound_ratio(x, ref, tol, stored_bf16=False) -> float:
    """max over elements of |x - ref| / (tol * rms(ref) + u * |ref|); must be <= 1."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    rms = float(np.sqrt(np.mean(ref * ref)))
    allow = tol * rms + (BF16_STORE if stored_bf16 else 0.0) * np.abs(ref)
    allow = np.maximum(allow, np.finfo(np.float64).tiny)
    return float(np.max(np.abs(x - ref) / allow))


def gated_bound_ratio(y, y_ref, gate, tol, stored_bf16=False) -> float:
    """Bound for the gated RMSNorm read-out y = n * gate, n = o / rms_row(o) (unit mean
    square per token and head), gate = w * silu(z) exact per element: the read-out
    bound tol, taken per row, carried through the gate factor, plus the bf16
    storage rounding of y itself (and of o, where the decode step's second pass
    reads the stored row):
        |y - y_ref| <= tol * |gate| + 2^-8 * |y_ref|
    Returns the max over elements of |y - y_ref| / allowance; must be <= 1."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    allow = tol * np.abs(np.asarray(gate, dtype=np.float64)) + (BF16_STORE if stored_bf16 else 0.0) * np.abs(y_ref)
    allow = np.maximum(allow, np.finfo(np.float64).tiny)
    return float(np.max(np.abs(y - y_ref) / allow))
