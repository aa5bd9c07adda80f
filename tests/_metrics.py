"""Error metrics for parity against the oracle.

Vector relative error: for every output vector (the last axis: one query row
of one head), max_c |g - o| / max_c |o|, then the maximum over vectors.  This
is the elementwise relative error made well-posed near zero entries.  For
scalars (lse) the error is |g - o| / max(1, |o|).
"""
import numpy as np


def vec_rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def scalar_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    d = np.where(both_inf, 0.0, np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0
