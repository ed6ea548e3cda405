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
# CGTP_ORACLE_LIB names another build of the oracle source (the mutation
# tests load deliberately broken copies this way, on the CPU only)
_LIB_PATH = os.environ.get("CGTP_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_ip = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if os.environ.get("CGTP_ORACLE_LIB"):
            raise RuntimeError(f"oracle library {_LIB_PATH} (CGTP_ORACLE_LIB) not found")
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
    lib.orc_sh_bwd.restype = None
    lib.orc_sh_bwd.argtypes = [ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp]
    lib.orc_node_grad.restype = None
    lib.orc_node_grad.argtypes = [ctypes.c_int64, ctypes.c_int64, _i64p, _i64p, _dp, _dp]
    lib.orc_conv_fwd.restype = ctypes.c_int
    lib.orc_conv_fwd.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 4
    lib.orc_conv_bwd.restype = ctypes.c_int
    lib.orc_conv_bwd.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 7
    lib.orc_conv_bwd_bwd.restype = ctypes.c_int
    lib.orc_conv_bwd_bwd.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 11
    lib.orc_cp_conv_fwd.restype = None
    lib.orc_cp_conv_fwd.argtypes = [ctypes.c_int] * 5 + [ctypes.c_int64, _i64p, _i64p] + [_dp] * 7
    lib.orc_cp_conv_bwd.restype = None
    lib.orc_cp_conv_bwd.argtypes = [ctypes.c_int] * 5 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 10
    lib.orc_conv_fwd_mid.restype = ctypes.c_int
    lib.orc_conv_fwd_mid.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64, _i64p, _i64p] + [_dp] * 4
    lib.orc_conv_bwd_mid.restype = ctypes.c_int
    lib.orc_conv_bwd_mid.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] * 2 + [_i64p, _i64p] + [_dp] * 7
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


def sh_bwd(L, r, dY):
    """Gradient of <dY, Y(r)> with respect to the edge vectors: [E][3]."""
    r = _f64(r).reshape(-1, 3)
    E = r.shape[0]
    dY = _f64(dY).reshape(E, (L + 1) ** 2)
    dr = np.zeros((E, 3))
    if E:
        _load().orc_sh_bwd(L, E, _p(r), _p(dY), _p(dr))
    return dr


def node_grad(row_ptr, src, dr):
    """Per-node gradient [N][3] from per-edge gradients of r = pos[src] - pos[dst]."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    N, E = row_ptr.shape[0] - 1, src.shape[0]
    dr = _f64(dr).reshape(E, 3)
    dpos = np.zeros((N, 3))
    _load().orc_node_grad(N, E, _p(row_ptr, _i64p), _p(src, _i64p), _p(dr), _p(dpos))
    return dpos


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


def mid_rows(l_in, l_sh, l_out):
    """Row count of the per-path outputs: sum over the paths of 2*l3+1."""
    return int(sum(2 * l3 + 1 for (_, _, l3) in paths(l_in, l_sh, l_out)))


def conv_fwd_mid(l_in, l_sh, l_out, row_ptr, src, x, Y, W):
    """Per-path outputs out_mid[N][D_mid][C] (path p owns 2*l3+1 rows, in path order)."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W = _f64(x), _f64(Y), _f64(W)
    N, C = x.shape[0], x.shape[2]
    out = np.zeros((N, mid_rows(l_in, l_sh, l_out), C))
    rc = _load().orc_conv_fwd_mid(l_in, l_sh, l_out, C, N, _p(row_ptr, _i64p), _p(src, _i64p), _p(x), _p(Y), _p(W),
                                  _p(out))
    if rc != 0:
        raise ValueError("oracle: unsupported degrees")
    return out


def conv_bwd_mid(l_in, l_sh, l_out, row_ptr, src, x, Y, W, G, want=("dx", "dW", "dY")):
    """(dx, dW, dY) of <G_mid, out_mid>; a gradient not in ``want`` is None."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W, G = _f64(x), _f64(Y), _f64(W), _f64(G)
    N, C = x.shape[0], x.shape[2]
    E = src.shape[0]
    dx = np.zeros_like(x) if "dx" in want else None
    dW = np.zeros_like(W) if "dW" in want else None
    dY = np.zeros_like(Y) if "dY" in want else None
    opt = lambda a: _p(a) if a is not None else None
    rc = _load().orc_conv_bwd_mid(l_in, l_sh, l_out, C, N, E, _p(row_ptr, _i64p), _p(src, _i64p), _p(x), _p(Y),
                                  _p(W), _p(G), opt(dx), opt(dW), opt(dY))
    if rc != 0:
        raise ValueError("oracle: unsupported degrees")
    return dx, dW, dY


def path_mix_fwd(l_in, l_sh, l_out, mid, Wmix):
    """Fully connected ("uvw") mixing of the per-path outputs: path p's block
    of 2*l3+1 rows is multiplied by its channel matrix Wmix[p] [C][C_out] and
    the paths of each l3 are summed (TDN rebuttal to cmnz: the fully connected
    CG tensor product).  mid [N][D_mid][C] -> out [N][(l_out+1)^2][C_out]."""
    mid, Wmix = _f64(mid), _f64(Wmix)
    N = mid.shape[0]
    out = np.zeros((N, (l_out + 1) ** 2, Wmix.shape[2]))
    o = 0
    for p, (l1, l2, l3) in enumerate(paths(l_in, l_sh, l_out)):
        d = 2 * l3 + 1
        for m in range(d):
            out[:, l3 * l3 + m, :] += mid[:, o + m, :] @ Wmix[p]
        o += d
    return out


def path_mix_bwd(l_in, l_sh, l_out, mid, Wmix, G):
    """(d_mid, d_Wmix) of <G, path_mix_fwd(mid, Wmix)>."""
    mid, Wmix, G = _f64(mid), _f64(Wmix), _f64(G)
    d_mid = np.zeros_like(mid)
    d_W = np.zeros_like(Wmix)
    o = 0
    for p, (l1, l2, l3) in enumerate(paths(l_in, l_sh, l_out)):
        d = 2 * l3 + 1
        for m in range(d):
            d_mid[:, o + m, :] = G[:, l3 * l3 + m, :] @ Wmix[p].T
            d_W[p] += mid[:, o + m, :].T @ G[:, l3 * l3 + m, :]
        o += d
    return d_mid, d_W


def conv_bwd_bwd(l_in, l_sh, l_out, row_ptr, src, x, Y, W, G, ggx=None, ggY=None, ggW=None,
                 want=("dx", "dY", "dW", "dG")):
    """Gradients (dx, dY, dW, dG) of S = <ggx, dx> + <ggW, dW> + <ggY, dY>
    with respect to x, Y, W and G, where (dx, dW, dY) = conv_bwd(x, Y, W, G);
    a cotangent given as None is zero, an output not in ``want`` is None."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W, G = _f64(x), _f64(Y), _f64(W), _f64(G)
    cot = [_f64(a) if a is not None else None for a in (ggx, ggY, ggW)]
    N, C = x.shape[0], x.shape[2]
    E = src.shape[0]
    dx = np.zeros_like(x) if "dx" in want else None
    dY = np.zeros_like(Y) if "dY" in want else None
    dW = np.zeros_like(W) if "dW" in want else None
    dG = np.zeros_like(G) if "dG" in want else None
    opt = lambda a: _p(a) if a is not None else None
    rc = _load().orc_conv_bwd_bwd(l_in, l_sh, l_out, C, N, E, _p(row_ptr, _i64p), _p(src, _i64p), _p(x), _p(Y),
                                  _p(W), _p(G), *(opt(a) for a in cot), opt(dx), opt(dY), opt(dW), opt(dG))
    if rc != 0:
        raise ValueError("oracle: unsupported degrees")
    return dx, dY, dW, dG


def conv_fwd_shared(l_in, l_sh, l_out, row_ptr, src, x, Y, Ws):
    """Forward with path-weight sharing: Ws [E][C] is every path's weight, so
    this is conv_fwd with W[e][p][u] = Ws[e][u] (TDN rebuttal to oXft: one
    weight matrix shared across paths)."""
    P = paths(l_in, l_sh, l_out).shape[0]
    Ws = _f64(Ws)
    return conv_fwd(l_in, l_sh, l_out, row_ptr, src, x, Y, np.repeat(Ws[:, None, :], P, axis=1))


def conv_bwd_shared(l_in, l_sh, l_out, row_ptr, src, x, Y, Ws, G, want=("dx", "dW", "dY")):
    """Backward with path-weight sharing: by the chain rule through
    W[e][p][u] = Ws[e][u], dWs[e][u] = sum over p of dW[e][p][u]."""
    P = paths(l_in, l_sh, l_out).shape[0]
    Ws = _f64(Ws)
    dx, dW, dY = conv_bwd(l_in, l_sh, l_out, row_ptr, src, x, Y, np.repeat(Ws[:, None, :], P, axis=1), G, want)
    return dx, (dW.sum(axis=1) if dW is not None else None), dY


def conv_bwd_bwd_shared(l_in, l_sh, l_out, row_ptr, src, x, Y, Ws, G, ggx=None, ggY=None, ggWs=None,
                        want=("dx", "dY", "dW", "dG")):
    """Double backward with path-weight sharing.  The shared backward returns
    dWs = sum over p of dW_p, so <ggWs, dWs> = <ggW, dW> with ggW[e][p][u] =
    ggWs[e][u] for every p; the gradient for Ws sums over the paths again."""
    P = paths(l_in, l_sh, l_out).shape[0]
    rep = lambda a: np.repeat(_f64(a)[:, None, :], P, axis=1) if a is not None else None
    dx, dY, dW, dG = conv_bwd_bwd(l_in, l_sh, l_out, row_ptr, src, x, Y, rep(Ws), G, ggx, ggY, rep(ggWs), want)
    return dx, dY, (dW.sum(axis=1) if dW is not None else None), dG


# ---------------------------------------------------------------------------
# CP-decomposed tensor product ("Tensor Decomposition Networks ...", rebuttal
# to S6y1: Equation (3), its gradients, and the data-free fit of the factors)
# ---------------------------------------------------------------------------
def cp_tensor(l_in, l_sh, l_out):
    """The whole coupling tensor M [d1][d2][d3] of the degree set: every
    path's real CG block T_p placed at the components of its degrees (a
    component triple belongs to at most one path), so that with one weight for
    every path the convolution couples x and y through M."""
    d1, d2, d3 = (l_in + 1) ** 2, (l_sh + 1) ** 2, (l_out + 1) ** 2
    M = np.zeros((d1, d2, d3))
    for l1, l2, l3 in paths(l_in, l_sh, l_out):
        M[l1 * l1:(l1 + 1) ** 2, l2 * l2:(l2 + 1) ** 2, l3 * l3:(l3 + 1) ** 2] = real_cg(l1, l2, l3)
    return M


def cp_exact_factors(M):
    """Factors of rank d1*d2 that reproduce M exactly: column r = (a, b) has
    B[:, r] = e_a, C[:, r] = e_b and A[:, r] = M[a, b, :]."""
    d1, d2, d3 = M.shape
    R = d1 * d2
    A, B, Cf = np.zeros((d3, R)), np.zeros((d1, R)), np.zeros((d2, R))
    for a in range(d1):
        for b in range(d2):
            r = a * d2 + b
            B[a, r] = 1.0
            Cf[b, r] = 1.0
            A[:, r] = M[a, b, :]
    return A, B, Cf


def cp_reconstruct(A, B, Cf):
    """The rank-R tensor sum_r B[:,r] (x) Cf[:,r] (x) A[:,r] as [d1][d2][d3]."""
    return np.einsum("ar,br,cr->abc", _f64(B), _f64(Cf), _f64(A))


def cp_objective(M, A, B, Cf):
    """Squared Frobenius error ||M - [[A, B, Cf]]||^2: the expected squared
    error of the approximate product over independent standard-normal x, y."""
    return float(((_f64(M) - cp_reconstruct(A, B, Cf)) ** 2).sum())


def cp_als_step(M, A, B, Cf, which, ridge=1e-12):
    """One ALS update: the factor `which` ("B", "C" or "A") replaced by the
    exact minimiser of the Frobenius error with the other two held fixed,
    K V^-1 with K the tensor contracted with the other two factors and V the
    Hadamard product of their Gram matrices (ridge * trace(V) / R added to
    V's diagonal).  Returns the new (A, B, Cf)."""
    M = _f64(M)
    R = A.shape[1]

    def solve(K, V):
        V = V + np.eye(R) * (ridge * np.trace(V) / R)
        return np.linalg.solve(V, K.T).T          # K V^-1 (V symmetric)

    if which == "B":
        B = solve(np.einsum("abc,br,cr->ar", M, Cf, A), (Cf.T @ Cf) * (A.T @ A))
    elif which == "C":
        Cf = solve(np.einsum("abc,ar,cr->br", M, B, A), (B.T @ B) * (A.T @ A))
    else:
        A = solve(np.einsum("abc,ar,br->cr", M, B, Cf), (B.T @ B) * (Cf.T @ Cf))
    return A, B, Cf


def cp_als(M, A, B, Cf, sweeps, ridge=1e-12):
    """Alternating least squares for the CP factors of M (the data-free fit:
    the Frobenius norm between exact and approximate product is minimised one
    factor at a time, each step an exact linear least-squares solve, see
    cp_als_step).  Order per sweep: B, then Cf, then A.  Returns (A, B, Cf,
    [relative error after each sweep])."""
    M = _f64(M)
    A, B, Cf = (np.array(_f64(v), copy=True) for v in (A, B, Cf))
    nrm = np.sqrt((M ** 2).sum())
    hist = []
    for _ in range(sweeps):
        for which in ("B", "C", "A"):
            A, B, Cf = cp_als_step(M, A, B, Cf, which, ridge)
        hist.append(np.sqrt(cp_objective(M, A, B, Cf)) / nrm)
    return A, B, Cf, hist


def cp_conv_fwd(row_ptr, src, x, Y, W, A, B, Cf):
    """out[N][d3][C] of the CP convolution: W [E][C] one weight per edge and
    channel, factors A [d3][R], B [d1][R], Cf [d2][R]."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W, A, B, Cf = (_f64(v) for v in (x, Y, W, A, B, Cf))
    N, d1, C = x.shape
    d3, R = A.shape
    d2 = Cf.shape[0]
    out = np.zeros((N, d3, C))
    _load().orc_cp_conv_fwd(d1, d2, d3, R, C, N, _p(row_ptr, _i64p), _p(src, _i64p), _p(x), _p(Y), _p(W), _p(A),
                            _p(B), _p(Cf), _p(out))
    return out


def cp_conv_bwd(row_ptr, src, x, Y, W, A, B, Cf, G, want=("dx", "dY", "dW")):
    """(dx, dY, dW) of <G, cp_conv_fwd(...)>; a gradient not in ``want`` is None."""
    row_ptr, src = _i64(row_ptr), _i64(src)
    x, Y, W, A, B, Cf, G = (_f64(v) for v in (x, Y, W, A, B, Cf, G))
    N, d1, C = x.shape
    d3, R = A.shape
    d2 = Cf.shape[0]
    E = src.shape[0]
    dx = np.zeros_like(x) if "dx" in want else None
    dY = np.zeros((E, d2)) if "dY" in want else None
    dW = np.zeros((E, C)) if "dW" in want else None
    opt = lambda a: _p(a) if a is not None else None
    _load().orc_cp_conv_bwd(d1, d2, d3, R, C, N, E, _p(row_ptr, _i64p), _p(src, _i64p), _p(x), _p(Y), _p(W),
                            _p(A), _p(B), _p(Cf), _p(G), opt(dx), opt(dY), opt(dW))
    return dx, dY, dW


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
