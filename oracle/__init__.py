"""fp64 CPU oracle for the CGTP convolution -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and the two
share no code: this is a thin ctypes wrapper over ``cgtp_oracle.c`` (plain C,
fp64, direct loops).

What each function computes, and the passage it follows, is stated in the C
source.  Arrays are numpy; every floating-point input is converted to float64
(exactly, for fp32 inputs) before the call and every output is float64.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_ip = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build_oracle
        build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_cg_complex.restype = ctypes.c_double
    lib.orc_cg_complex.argtypes = [ctypes.c_int] * 6
    lib.orc_real_cg_parts.restype = None
    lib.orc_real_cg_parts.argtypes = [ctypes.c_int] * 3 + [_dp, _dp]
    lib.orc_real_cg.restype = None
    lib.orc_real_cg.argtypes = [ctypes.c_int] * 3 + [_dp]
    lib.orc_paths.restype = ctypes.c_int
    lib.orc_paths.argtypes = [ctypes.c_int] * 3 + [_ip]
    lib.orc_sh.restype = None
    lib.orc_sh.argtypes = [ctypes.c_int, ctypes.c_int64, _dp, _dp]
    lib.orc_conv_fwd.restype = ctypes.c_int
    lib.orc_conv_fwd.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 4
    lib.orc_conv_bwd.restype = ctypes.c_int
    lib.orc_conv_bwd.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 7
    lib.orc_graph_transpose.restype = None
    lib.orc_graph_transpose.argtypes = [ctypes.c_int64, ctypes.c_int64, _i64p, _i64p, _i64p, _i64p, _i64p]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _i64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def _p(a, t=_dp):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().orc_num_threads())


def cg_complex(j1, m1, j2, m2, J, M) -> float:
    """<j1 m1 j2 m2 | J M>, complex basis, Condon-Shortley phase (Racah's formula)."""
    return float(_load().orc_cg_complex(j1, m1, j2, m2, J, M))


def real_cg_parts(l1, l2, l3):
    """(Re S, Im S) of the real-basis coupling tensor, each [2l1+1][2l2+1][2l3+1]."""
    shape = (2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)
    re = np.zeros(shape)
    im = np.zeros(shape)
    _load().orc_real_cg_parts(l1, l2, l3, _p(re), _p(im))
    return re, im


def real_cg(l1, l2, l3):
    """Real CG tensor T_p [2l1+1][2l2+1][2l3+1] (Re S for even l1+l2+l3, Im S for odd)."""
    T = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    _load().orc_real_cg(l1, l2, l3, _p(T))
    return T


def paths(l_in, l_sh, l_out):
    """[P][3] int array of (l1, l2, l3) in lexicographic order."""
    lib = _load()
    P = lib.orc_paths(l_in, l_sh, l_out, None)
    out = np.zeros((P, 3), dtype=np.int32)
    lib.orc_paths(l_in, l_sh, l_out, out.ctypes.data_as(_ip))
    return out.astype(np.int64)


def sh(L, r):
    """Real spherical harmonics of degrees 0..L of r/|r|; r [E][3] -> Y [E][(L+1)^2]."""
    r = _f64(r).reshape(-1, 3)
    E = r.shape[0]
    Y = np.zeros((E, (L + 1) ** 2))
    if E:
        _load().orc_sh(L, E, _p(r), _p(Y))
    return Y


def conv_fwd(l_in, l_sh, l_out, row_ptr, src, x, Y, W):
    """out[N][D_out][C] of the CGTP convolution over a receiver-sorted CSR."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W = _f64(x), _f64(Y), _f64(W)
    N, C = x.shape[0], x.shape[2]
    E = src.shape[0]
    out = np.zeros((N, (l_out + 1) ** 2, C))
    rc = _load().orc_conv_fwd(l_in, l_sh, l_out, C, N, E, _p(row_ptr, _i64p), _p(src, _i64p),
                              _p(x), _p(Y), _p(W), _p(out))
    if rc != 0:
        raise ValueError("oracle: unsupported degrees")
    return out


def conv_bwd(l_in, l_sh, l_out, row_ptr, src, x, Y, W, G, want=("dx", "dW", "dY")):
    """(dx, dW, dY) of L = <G, out>; a gradient not in ``want`` is returned as None."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W, G = _f64(x), _f64(Y), _f64(W), _f64(G)
    N, C = x.shape[0], x.shape[2]
    E = src.shape[0]
    dx = np.zeros_like(x) if "dx" in want else None
    dW = np.zeros_like(W) if "dW" in want else None
    dY = np.zeros_like(Y) if "dY" in want else None
    rc = _load().orc_conv_bwd(l_in, l_sh, l_out, C, N, E, _p(row_ptr, _i64p), _p(src, _i64p),
                              _p(x), _p(Y), _p(W), _p(G),
                              _p(dx) if dx is not None else None,
                              _p(dW) if dW is not None else None,
                              _p(dY) if dY is not None else None)
    if rc != 0:
        raise ValueError("oracle: unsupported degrees")
    return dx, dW, dY


def graph_transpose(row_ptr, src):
    """(srow_ptr[N+1], perm[E], sdst[E]): edges stably grouped by sender."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    N, E = row_ptr.shape[0] - 1, src.shape[0]
    srow = np.zeros(N + 1, dtype=np.int64)
    perm = np.zeros(E, dtype=np.int64)
    sdst = np.zeros(E, dtype=np.int64)
    _load().orc_graph_transpose(N, E, _p(row_ptr, _i64p), _p(src, _i64p), _p(srow, _i64p),
                                _p(perm, _i64p), _p(sdst, _i64p))
    return srow, perm, sdst
