"""Rotation helpers for the equivariance pins (test code, fp64).

The real Wigner-D matrix of degree l is fitted from the oracle's spherical
harmonics: for sample directions v_k, Y_l(R v_k) = D_l(R) Y_l(v_k), solved by
least squares over 4(2l+1) directions.  It depends only on the spherical
harmonics, which are pinned separately (scipy, addition theorem), so it can
check the CG tables and the convolution without sharing their code.
"""
import math

import numpy as np


def unit_vectors(n, seed):
    rng = np.random.default_rng([seed, 99])
    v = rng.normal(size=(n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def wigner_d_real(oracle, l, R, seed=0):
    """D_l(R), (2l+1)x(2l+1), with Y_l(R v) = D_l(R) Y_l(v)."""
    L = l
    v = unit_vectors(4 * (2 * l + 1) + 8, seed)
    Y = oracle.sh(L, v)[:, l * l:(l + 1) ** 2]
    Yr = oracle.sh(L, v @ R.T)[:, l * l:(l + 1) ** 2]
    Dt, *_ = np.linalg.lstsq(Y, Yr, rcond=None)
    return Dt.T


def block_diag_d(oracle, L, R, seed=0):
    """Block-diagonal D over degrees 0..L, acting on a [(L+1)^2] component vector."""
    D = np.zeros(((L + 1) ** 2, (L + 1) ** 2))
    for l in range(L + 1):
        D[l * l:(l + 1) ** 2, l * l:(l + 1) ** 2] = wigner_d_real(oracle, l, R, seed)
    return D


def complex_to_real(l):
    """Unitary U with Y_real = U Y_complex, written from the real-SH definition
    Y_{l,m} = sqrt2 (-1)^m Im Y_l^{|m|} (m<0), Y_l^0 (m=0), sqrt2 (-1)^m Re Y_l^m (m>0)."""
    d = 2 * l + 1
    U = np.zeros((d, d), dtype=complex)
    s = 1 / math.sqrt(2)
    for m in range(-l, l + 1):
        if m == 0:
            U[l, l] = 1
        elif m > 0:
            U[m + l, m + l] = (-1) ** m * s
            U[m + l, -m + l] = s
        else:
            U[m + l, m + l] = 1j * s
            U[m + l, -m + l] = -1j * (-1) ** m * s
    return U
