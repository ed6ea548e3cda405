"""GPU parity of the CP-decomposed tensor-product convolution
(cgtp_cp_conv_fwd / cgtp_cp_conv_bwd) against the oracle.

The oracle's CP convolution is pinned on the CPU (exact factors reproduce the
pinned convolution with one weight for every path; its backward by exact
finite differences).  Here the HIP path is compared with it element by
element on seeded inputs: every padded rank (16, 32, 64) with ragged ranks
inside each, every lane geometry (16, 32, 64 lanes per node, two waves per
node), degrees up to 3 and mixed, a graph many rounds of blocks deep, empty
graphs, partial gradients, and factors from the library's own fit.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import synth
from tests.metrics import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _log(*a):
    print(*a, flush=True)


def _graph(N, seed, max_deg=12):
    rng = np.random.default_rng(seed)
    degs = rng.integers(0, max_deg, size=N)
    if N > 40:
        degs[[0, 5, 6, 33]] = 0
        degs[8] = N - 1
        degs[9] = 17
    return synth.random_graph(N, degs, seed=seed + 1)


def run_cp(torch, dev, oracle, Ls, C, R, N=70, seed=0, factors=None, want=("dx", "dW", "dY"), max_deg=12):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    li, ls, lo = Ls
    g = _graph(N, seed=li * 1000 + ls * 100 + lo * 10 + C + R + seed, max_deg=max_deg)
    E = g.n_edges
    plan = Plan(li, ls, lo, C)
    d1, d2, d3 = plan.dim_in, plan.dim_sh, plan.dim_out
    rng = np.random.default_rng(seed + 31)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x, W, G = f(N, d1, C), f(E, C), f(N, d3, C)
    if factors is None:
        A, B, Cf = f(d3, R), f(d1, R), f(d2, R)
    else:
        A, B, Cf = (np.ascontiguousarray(v, dtype=np.float32) for v in factors)
        R = A.shape[1]
    Y = oracle.sh(ls, g.r).astype(np.float32)
    _log(f"[cp] {Ls} C={C} R={R} N={N} E={E} want={want}")
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    args = (rp, sr, T(x), T(Y), T(W), T(A), T(B), T(Cf))
    out = plan.cp_conv_fwd(*args).cpu().numpy()
    dx, dW, dY = (t.cpu().numpy() if t is not None else None for t in plan.cp_conv_bwd(*args, T(G), want=want))
    ro = oracle.cp_conv_fwd(g.row_ptr, g.src, x, Y, W, A, B, Cf)
    rdx, rdY, rdW = oracle.cp_conv_bwd(g.row_ptr, g.src, x, Y, W, A, B, Cf, G)
    assert_parity(out, ro, "out")
    for name, key, u, v in (("dx", "dx", dx, rdx), ("dW", "dW", dW, rdW), ("dY", "dY", dY, rdY)):
        if key in want:
            assert_parity(u, v, name)
        else:
            assert u is None
    return g, (x, Y, W, G), out, (dx, dW, dY)


# every padded rank x every lane geometry, ragged ranks and channel counts
CASES = [((2, 2, 2), C, R) for C in (8, 16, 24, 32, 48, 64, 100, 128) for R in (5, 16, 17, 32, 40, 64)]


@pytest.mark.parametrize("Ls,C,R", CASES)
def test_cp_every_rank_and_geometry(torch_dev, oracle, Ls, C, R):
    torch, dev = torch_dev
    g, _, out, (dx, _, _) = run_cp(torch, dev, oracle, Ls, C, R)
    assert np.all(out[[0, 5, 6, 33]] == 0)
    no_out = np.setdiff1d(np.arange(g.n_nodes), g.src)
    assert np.all(dx[no_out] == 0)


@pytest.mark.parametrize("Ls,C,R", [((1, 1, 1), 1, 1), ((3, 3, 3), 64, 48), ((3, 3, 3), 128, 64), ((3, 3, 3), 16, 20),
                                    ((2, 1, 3), 32, 12), ((3, 2, 1), 96, 33), ((0, 1, 1), 64, 3), ((1, 2, 0), 128, 7)])
def test_cp_degrees(torch_dev, oracle, Ls, C, R):
    torch, dev = torch_dev
    run_cp(torch, dev, oracle, Ls, C, R)


@pytest.mark.parametrize("Ls,C", [((1, 1, 1), 64), ((2, 1, 1), 128), ((1, 1, 0), 16)])
def test_cp_exact_factors_give_the_exact_convolution(torch_dev, oracle, Ls, C):
    """Factors that represent the coupling tensor exactly (rank d1*d2 <= 64):
    parity with the oracle's CP convolution on the same (fp32) factors, and
    the exact convolution with one weight for every path to within the fp32
    rounding of the factors (the CG values in A are not fp32 numbers, so only
    the whole-tensor error is bounded: relative L2 <= 1e-6)."""
    torch, dev = torch_dev
    factors = oracle.cp_exact_factors(oracle.cp_tensor(*Ls))
    g, (x, Y, W, G), out, (dx, dW, dY) = run_cp(torch, dev, oracle, Ls, C, 0, factors=factors)
    rel = lambda u, v: np.linalg.norm(u - v) / np.linalg.norm(v)
    assert rel(out, oracle.conv_fwd_shared(*Ls, g.row_ptr, g.src, x, Y, W)) <= 1e-6
    rdx, rdW, rdY = oracle.conv_bwd_shared(*Ls, g.row_ptr, g.src, x, Y, W, G)
    assert rel(dx, rdx) <= 1e-6 and rel(dW, rdW) <= 1e-6 and rel(dY, rdY) <= 1e-6


def test_cp_fitted_factors(torch_dev, oracle):
    """Factors from the library's own data-free fit (degree 2, rank 64, where
    the fit is exact to ~1e-6): parity with the oracle's CP convolution on
    the same factors, and closeness to the exact convolution within the fit's
    error."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    Ls, C, R = (2, 2, 2), 64, 64
    plan = Plan(*Ls, C)
    rng = np.random.default_rng(11)
    A, B, Cf, err = plan.cp_fit(rng.standard_normal((9, R)), rng.standard_normal((9, R)),
                                rng.standard_normal((9, R)), sweeps=300)
    assert err < 1e-5
    g, (x, Y, W, G), out, _ = run_cp(torch, dev, oracle, Ls, C, R, factors=(A, B, Cf))
    exact = oracle.conv_fwd_shared(*Ls, g.row_ptr, g.src, x, Y, W)
    assert np.linalg.norm(out - exact) <= 1e-4 * np.linalg.norm(exact)


@pytest.mark.parametrize("want", [("dx",), ("dW",), ("dY",), ("dW", "dY")])
def test_cp_partial_gradients(torch_dev, oracle, want):
    torch, dev = torch_dev
    run_cp(torch, dev, oracle, (2, 2, 2), 100, 40, want=want)


@pytest.mark.parametrize("C,R", [(128, 32), (64, 64), (16, 16)])
def test_cp_many_nodes(torch_dev, oracle, C, R):
    """A grid many rounds of blocks deep with short ragged segments."""
    torch, dev = torch_dev
    run_cp(torch, dev, oracle, (2, 2, 2), C, R, N=5003, max_deg=7)


def test_cp_empty_graph(torch_dev):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64)
    f = lambda *s: torch.randn(*s, device=dev)
    A, B, Cf = f(9, 16), f(9, 16), f(9, 16)
    for N in (9, 1):
        rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        sr = torch.zeros(0, dtype=torch.int32, device=dev)
        x, G = f(N, 9, 64), f(N, 9, 64)
        Y, W = torch.zeros(0, 9, device=dev), torch.zeros(0, 64, device=dev)
        out = plan.cp_conv_fwd(rp, sr, x, Y, W, A, B, Cf)
        dx, dW, dY = plan.cp_conv_bwd(rp, sr, x, Y, W, A, B, Cf, G)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out) == 0 and torch.count_nonzero(dx) == 0
        assert dW.shape == (0, 64) and dY.shape == (0, 9)
