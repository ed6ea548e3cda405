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


class WholeTensor:
    """The parity metric of one whole output tensor, accumulated over chunks.

    The GPU tensor stays on the device; each chunk of it is compared with the
    oracle's fp64 values for the same entries (moved to the device; the
    arithmetic of the comparison runs in torch fp64).  Sums of squared errors
    and of squared reference values give the exact whole-tensor relative L2
    error.  The elementwise criterion needs the threshold FLOOR * ||r||
    before ||r|| is known, so chunks are checked against the lower threshold
    FLOOR * ||g|| * (1 - 1e-4) (||g||: the whole GPU tensor's norm), a superset
    of the entries the criterion names whenever the relative L2 error is
    below 1e-5 (then ||r|| >= ||g|| (1 - 1e-5)); check() asserts that this
    held.
    """

    def __init__(self, torch, gpu_tensor, name, chunk=1 << 26):
        self.torch, self.name, self.chunk = torch, name, chunk
        self.gnorm = self.norm(gpu_tensor)
        self.thr = FLOOR * self.gnorm * (1.0 - 1e-4)
        self.d2 = 0.0
        self.r2 = 0.0
        self.max_rel = 0.0
        self.n = 0
        self.n_checked = 0
        self.finite = True

    def dot(self, a, b):
        """fp64 sum of a*b over two whole device tensors, in chunks."""
        a, b = a.reshape(-1), b.reshape(-1)
        tot = 0.0
        for k in range(0, a.numel(), self.chunk):
            tot += float((a[k:k + self.chunk].double() * b[k:k + self.chunk].double()).sum())
        return tot

    def norm(self, a):
        return self.dot(a, a) ** 0.5

    def add(self, g, r):
        """g: device tensor (a slice of the GPU result); r: the oracle's fp64
        values of the same entries (numpy, same shape)."""
        torch = self.torch
        g = g.reshape(-1)
        r = np.ascontiguousarray(r, dtype=np.float64).reshape(-1)
        assert g.numel() == r.shape[0], (self.name, g.numel(), r.shape)
        for k in range(0, r.shape[0], self.chunk):
            gg = g[k:k + self.chunk].double()
            rr = torch.from_numpy(r[k:k + self.chunk]).to(gg.device)
            self.finite = self.finite and bool(torch.isfinite(gg).all())
            d = gg - rr
            self.d2 += float((d * d).sum())
            self.r2 += float((rr * rr).sum())
            big = rr.abs() > self.thr
            nb = int(big.sum())
            if nb:
                self.max_rel = max(self.max_rel, float((d[big].abs() / rr[big].abs()).max()))
            self.n += rr.numel()
            self.n_checked += nb

    def check(self):
        rn = self.r2 ** 0.5
        rel_l2 = (self.d2 ** 0.5) / rn if rn > 0 else self.d2 ** 0.5
        m = {"rel_l2": rel_l2, "max_rel": self.max_rel, "n": self.n, "n_checked": self.n_checked}
        print(f"[whole] {self.name}: {m}", flush=True)
        assert self.finite, f"{self.name}: non-finite values in GPU result"
        assert self.thr <= FLOOR * rn, f"{self.name}: checked set does not cover the criterion ({m})"
        assert rel_l2 <= REL_L2 and self.max_rel <= MAX_REL, f"{self.name}: {m}"
        return m
