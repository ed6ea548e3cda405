"""Parity metric between a GPU result g and the fp64 oracle r.

Per output tensor: relative L2 error ||g - r|| / ||r|| <= 1e-5, and the largest
elementwise relative error |g_k - r_k| / |r_k| over the entries with
|r_k| > 1e-6 ||r|| must be <= 1e-4.  When only a sample of the entries is
checked, ``norm`` is the L2 norm of the whole tensor (taken from the GPU
result) and the relative L2 error is that of the sample.
"""
import numpy as np

REL_L2 = 1e-5
MAX_REL = 1e-4
FLOOR = 1e-6


def parity(g, r, norm=None):
    g = np.asarray(g, dtype=np.float64).ravel()
    r = np.asarray(r, dtype=np.float64).ravel()
    assert g.shape == r.shape
    rn = float(np.linalg.norm(r))
    full = rn if norm is None else float(norm)
    d = np.abs(g - r)
    rel_l2 = float(np.linalg.norm(g - r) / rn) if rn > 0 else float(np.linalg.norm(g))
    big = np.abs(r) > FLOOR * full
    max_rel = float((d[big] / np.abs(r[big])).max()) if big.any() else 0.0
    return {"rel_l2": rel_l2, "max_rel": max_rel, "n": int(r.size), "n_checked": int(big.sum())}


def assert_parity(g, r, name, norm=None):
    m = parity(g, r, norm)
    if not np.all(np.isfinite(np.asarray(g, dtype=np.float64))):
        raise AssertionError(f"{name}: non-finite values in GPU result")
    assert m["rel_l2"] <= REL_L2 and m["max_rel"] <= MAX_REL, f"{name}: {m}"
    return m
