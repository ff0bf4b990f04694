"""Shared test helpers: golden-fixture reader and the elementwise error metric."""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse a tests/golden/*.txt fixture: '#' comments, then 'key value value ...' lines."""
    out = {}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "kind":
                out[key] = vals[0]
            elif key in ("m", "n", "ldx"):
                out[key] = int(vals[0])
            elif key in ("alpha", "beta"):
                out[key] = float(vals[0])
            elif key in ("row_ptr", "col_idx"):
                out[key] = np.array([int(x) for x in vals], dtype=np.int32)
            elif key.startswith("expected"):
                out[key] = np.array([float(x) for x in vals], dtype=np.float64)
            else:
                out[key] = np.array([float(x) for x in vals], dtype=np.float32)
    return out


def golden_names():
    return sorted(f for f in os.listdir(GOLDEN_DIR) if f.endswith(".txt"))


def max_rel_err(out, ref, bound) -> float:
    """max_j |out_j - ref_j| / D_j with D_j the oracle's absolute-value bound.

    Entries with D_j == 0 must be exactly 0 (they count as error inf otherwise);
    non-finite reference entries must be matched in kind (NaN for NaN, same-signed Inf).
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    fin = np.isfinite(ref)
    if not np.array_equal(np.isnan(out), np.isnan(ref)):
        return math.inf
    inf_ref = np.isinf(ref)
    if not np.array_equal(out[inf_ref], ref[inf_ref]) or np.isinf(out[fin]).any():
        return math.inf
    o, r, d = out[fin], ref[fin], bound[fin]
    zero = d == 0
    if np.any(o[zero] != 0):
        return math.inf
    if not np.any(~zero):
        return 0.0
    return float(np.max(np.abs(o[~zero] - r[~zero]) / d[~zero]))
