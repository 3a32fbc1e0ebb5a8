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


def _rows2d(x):
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-1]) if x.ndim > 1 else x.reshape(-1, 1)


def worst_row_rel(x, ref, floor_frac: float = 0.05) -> float:
    """Largest relative L2 error of a single row (the last axis): the row's
    error norm over its reference norm, the latter taken at least floor_frac
    times the RMS row norm of the reference (rows that are zero in exact
    arithmetic are measured against a typical row instead)."""
    a, b = _rows2d(x), _rows2d(ref)
    nb = np.linalg.norm(b, axis=1)
    floor = floor_frac * float(np.sqrt(np.mean(nb ** 2))) if nb.size else 0.0
    den = np.maximum(nb, floor)
    err = np.linalg.norm(a - b, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(den > 0, err / np.where(den > 0, den, 1.0), err)
    return float(np.max(r)) if r.size else 0.0


def worst_tile_rel(x, ref, tile_rows: int = 64, floor_frac: float = 0.05) -> float:
    """Largest relative L2 error of one tile of tile_rows consecutive rows
    (along the second-to-last axis, per index of the leading axes; a ragged
    last tile is shorter) by the whole last axis, with the same floor as
    worst_row_rel applied to the tile norms."""
    a = np.asarray(x, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    if a.ndim < 2:
        a, b = a.reshape(-1, 1), b.reshape(-1, 1)
    n, c = a.shape[-2], a.shape[-1]
    a, b = a.reshape(-1, n, c), b.reshape(-1, n, c)
    errs, norms = [], []
    for i0 in range(0, n, tile_rows):
        d = a[:, i0:i0 + tile_rows] - b[:, i0:i0 + tile_rows]
        errs.append(np.sqrt(np.sum(d * d, axis=(1, 2))))
        norms.append(np.sqrt(np.sum(b[:, i0:i0 + tile_rows] ** 2, axis=(1, 2))))
    e, nb = np.concatenate(errs), np.concatenate(norms)
    floor = floor_frac * float(np.sqrt(np.mean(nb ** 2)))
    den = np.maximum(nb, floor)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(den > 0, e / np.where(den > 0, den, 1.0), e)
    return float(np.max(r))
