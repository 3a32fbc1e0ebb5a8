"""Accuracy metrics named on the SageAttention3 summary page ("Experimental
setup": CosSim, L1, RMSE), computed over the whole flattened tensor in float64.
Test infrastructure only."""
import numpy as np


def _flat(x):
    return np.asarray(x, dtype=np.float64).ravel()


def cos_sim(x, y) -> float:
    a, b = _flat(x), _flat(y)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def rel_l2(x, ref) -> float:
    a, b = _flat(x), _flat(ref)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    return float(d / nb) if nb > 0 else float(d)


def l1(x, ref) -> float:
    """Mean absolute error relative to the mean magnitude of the reference."""
    a, b = _flat(x), _flat(ref)
    den = np.mean(np.abs(b))
    return float(np.mean(np.abs(a - b)) / den) if den > 0 else float(np.mean(np.abs(a - b)))


def rmse(x, ref) -> float:
    a, b = _flat(x), _flat(ref)
    return float(np.sqrt(np.mean((a - b) ** 2)))
