"""Pins of the oracle's spherical-harmonics backward and per-node gradient.

The backward's grad_Y term feeds the forces of an interatomic potential
(the AccelNet review, Referee Report, validates analytic forces by finite
differences).  The pages give no formula, so the
pins are the mathematics: central finite differences of independently
computed spherical harmonics (scipy's complex SH through the change of
basis), the SH depending on the direction only (tangency, scale), rotation
covariance through Wigner-D matrices, a brute-force scatter, and finite
differences of the whole chain positions -> edge vectors -> SH -> CGTP
convolution -> <G, out>.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd.synth import random_rotation
from tests.rotations import block_diag_d, complex_to_real
from tests.test_oracle_sh import _scipy_complex_sh


def scipy_real_sh(L, r):
    """Real SH of degrees 0..L from scipy's complex SH (independent of the oracle)."""
    blocks = []
    for l in range(L + 1):
        blocks.append((complex_to_real(l) @ _scipy_complex_sh(l, r).T).T.real)
    return np.concatenate(blocks, axis=1)


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_sh_bwd_is_the_derivative_of_scipy_sh(oracle, L):
    rng = np.random.default_rng(L)
    r = rng.normal(size=(40, 3)) * rng.uniform(0.5, 4.0, size=(40, 1))
    dY = rng.normal(size=(40, (L + 1) ** 2))
    got = oracle.sh_bwd(L, r, dY)
    h = 1e-5
    want = np.zeros_like(got)
    for a in range(3):
        d = np.zeros(3)
        d[a] = h
        fp = (scipy_real_sh(L, r + d) * dY).sum(axis=1)
        fm = (scipy_real_sh(L, r - d) * dY).sum(axis=1)
        want[:, a] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


def test_sh_bwd_depends_on_the_direction_only(oracle):
    rng = np.random.default_rng(3)
    r = rng.normal(size=(60, 3))
    dY = rng.normal(size=(60, 16))
    g = oracle.sh_bwd(3, r, dY)
    # no radial component, and a 1/|r| scale
    np.testing.assert_allclose((g * r).sum(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(oracle.sh_bwd(3, 2.5 * r, dY), g / 2.5, rtol=1e-13, atol=1e-15)
    # degree 0 is constant
    assert np.all(oracle.sh_bwd(0, r, dY[:, :1]) == 0.0)


def test_sh_bwd_rotation_covariance(oracle):
    """<D dY, Y(R r)> = <dY, Y(r)>, so grad(R r, D dY) = R grad(r, dY)."""
    rng = np.random.default_rng(4)
    r = rng.normal(size=(30, 3))
    dY = rng.normal(size=(30, 16))
    for seed in range(3):
        R = random_rotation(seed)
        D = block_diag_d(oracle, 3, R)
        np.testing.assert_allclose(oracle.sh_bwd(3, r @ R.T, dY @ D.T), oracle.sh_bwd(3, r, dY) @ R.T,
                                   rtol=1e-10, atol=1e-11)


def test_node_grad_is_the_signed_scatter(oracle):
    from clebsch_gordan_tensor_cgtp_amd.synth import random_graph
    rng = np.random.default_rng(5)
    N = 40
    g = random_graph(N, rng.integers(0, 8, size=N), seed=6)
    dr = rng.normal(size=(g.n_edges, 3))
    want = np.zeros((N, 3))
    recv = np.repeat(np.arange(N), np.diff(g.row_ptr))
    np.add.at(want, g.src, dr)
    np.add.at(want, recv, -dr)
    np.testing.assert_allclose(oracle.node_grad(g.row_ptr, g.src, dr), want, atol=1e-14)


def _cluster(n, seed, rc=2.6):
    """Atoms in open space (no periodic images) and their cutoff graph,
    receiver-sorted, r = pos[sender] - pos[receiver]."""
    rng = np.random.default_rng(seed)
    pos = rng.uniform(0, 4.5, size=(n, 3))
    recv, send = [], []
    for i in range(n):
        for j in range(n):
            if i != j and np.linalg.norm(pos[j] - pos[i]) < rc:
                recv.append(i)
                send.append(j)
    recv, send = np.array(recv), np.array(send)
    row_ptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(recv, minlength=n), out=row_ptr[1:])
    return pos, row_ptr, send


@pytest.mark.parametrize("L", [1, 2, 3])
def test_forces_match_finite_differences_of_the_energy(oracle, L):
    """S(pos) = <G, out(x, Y(pos[src] - pos[dst]), W)>; its gradient with
    respect to every atom position, from conv_bwd's grad_Y through sh_bwd and
    node_grad, against central differences of S."""
    n, C = 14, 3
    pos, row_ptr, src = _cluster(n, seed=L)
    E = src.shape[0]
    recv = np.repeat(np.arange(n), np.diff(row_ptr))
    P = oracle.paths(L, L, L).shape[0]
    rng = np.random.default_rng(10 + L)
    x = rng.normal(size=(n, (L + 1) ** 2, C))
    W = rng.normal(size=(E, P, C))
    G = rng.normal(size=(n, (L + 1) ** 2, C))

    def energy(p):
        Y = oracle.sh(L, p[src] - p[recv])
        return float((G * oracle.conv_fwd(L, L, L, row_ptr, src, x, Y, W)).sum())

    r = pos[src] - pos[recv]
    _, _, dY = oracle.conv_bwd(L, L, L, row_ptr, src, x, oracle.sh(L, r), W, G, want=("dY",))
    grad = oracle.node_grad(row_ptr, src, oracle.sh_bwd(L, r, dY))
    h = 1e-5
    fd = np.zeros_like(grad)
    for k in range(n):
        for a in range(3):
            p = pos.copy()
            p[k, a] += h
            ep = energy(p)
            p[k, a] -= 2 * h
            fd[k, a] = (ep - energy(p)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7 * np.abs(fd).max())
    # translation invariance: the forces sum to zero
    np.testing.assert_allclose(grad.sum(axis=0), 0.0, atol=1e-12 * np.abs(grad).max())
