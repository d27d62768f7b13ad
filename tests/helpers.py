"""Comparison rules shared by the tests (no attention arithmetic here)."""
import numpy as np


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Worst per-row error max_d|got - ref| / max_d|ref| over rows with a nonzero reference.

    Rows whose reference is exactly 0 (an empty visible set) must be exactly 0 in
    ``got``; any other value there is reported as an infinite error.
    """
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    if np.any(zero) and np.any(got[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    num = np.abs(got[~zero] - ref[~zero]).max(axis=1)
    return float((num / den[~zero]).max())
