"""GPU parity of the per-path (concatenated) outputs (CGTP_FLAG_PATH_OUTPUTS)
against the oracle.

The oracle's per-path convolution is pinned on the CPU against the summed
convolution (its blocks sum to it per l3) and by finite differences.  Here
the HIP path (a forward launch per group of paths, a backward that reads
each path's own block of grad_out) is compared with it element by element:
every lane geometry and channel-count class, every degree up to 3 (one to
eleven path groups), mixed degrees, path-weight sharing, a grid many rounds
of blocks deep and empty graphs.
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


def run_mid(torch, dev, oracle, li, ls, lo, C, N=70, seed=0, shared=False, max_deg=12):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    g = _graph(N, seed=li * 1000 + ls * 100 + lo * 10 + C + seed, max_deg=max_deg)
    E = g.n_edges
    plan = Plan(li, ls, lo, C, shared_weights=shared, path_outputs=True)
    P = len(plan.paths)
    D = plan.dim_out
    assert D == oracle.mid_rows(li, ls, lo)
    rng = np.random.default_rng(seed + 7)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x, G = f(N, (li + 1) ** 2, C), f(N, D, C)
    W = f(E, plan.weight_rows, C)
    Y = oracle.sh(ls, g.r).astype(np.float32)
    _log(f"[mid] ({li},{ls},{lo}) C={C} N={N} E={E} shared={shared} D_mid={D}")
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    out = plan.conv_fwd(rp, sr, T(x), T(Y), T(W)).cpu().numpy()
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G)))
    Wfull = np.repeat(W, P, axis=1) if shared else W
    ro = oracle.conv_fwd_mid(li, ls, lo, g.row_ptr, g.src, x, Y, Wfull)
    rdx, rdW, rdY = oracle.conv_bwd_mid(li, ls, lo, g.row_ptr, g.src, x, Y, Wfull, G)
    if shared:
        rdW = rdW.sum(axis=1, keepdims=True)
    assert_parity(out, ro, "out")
    assert_parity(dx, rdx, "dx")
    assert_parity(dW, rdW, "dW")
    assert_parity(dY, rdY, "dY")
    return g, out, dx


CHANNELS = (1, 8, 24, 64, 100, 128)


@pytest.mark.parametrize("L,C", [(L, C) for L in (1, 2, 3) for C in CHANNELS])
def test_path_outputs_every_geometry(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    g, out, dx = run_mid(torch, dev, oracle, L, L, L, C)
    assert np.all(out[[0, 5, 6, 33]] == 0)
    no_out = np.setdiff1d(np.arange(g.n_nodes), g.src)
    assert np.all(dx[no_out] == 0)


@pytest.mark.parametrize("li,ls,lo,C", [(2, 1, 3, 24), (3, 2, 1, 64), (1, 3, 2, 96), (0, 1, 1, 16), (2, 2, 0, 8),
                                        (3, 3, 2, 128), (0, 0, 0, 32)])
def test_path_outputs_mixed_degrees(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_mid(torch, dev, oracle, li, ls, lo, C)


@pytest.mark.parametrize("li,ls,lo,C", [(2, 2, 2, 128), (3, 3, 3, 64), (1, 2, 2, 16)])
def test_path_outputs_with_shared_weights(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_mid(torch, dev, oracle, li, ls, lo, C, shared=True)


@pytest.mark.parametrize("L,C", [(2, 128), (3, 64), (1, 16)])
def test_path_outputs_many_nodes(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    run_mid(torch, dev, oracle, L, L, L, C, N=5003, max_deg=7)


def test_path_outputs_empty_graph_and_unsupported_double_backward(torch_dev):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd import _lib
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64, path_outputs=True)
    N = 9
    rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    sr = torch.zeros(0, dtype=torch.int32, device=dev)
    x = torch.randn(N, 9, 64, device=dev)
    Y = torch.zeros(0, 9, device=dev)
    W = torch.zeros(0, 15, 64, device=dev)
    out = plan.conv_fwd(rp, sr, x, Y, W)
    dx, dW, dY = plan.conv_bwd(rp, sr, x, Y, W, torch.randn(N, 51, 64, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (N, 51, 64) and torch.count_nonzero(out) == 0 and torch.count_nonzero(dx) == 0
    with pytest.raises(_lib.CgtpError) as ei:
        plan.conv_bwd_bwd(rp, sr, x, Y, W, out)
    assert ei.value.status == _lib.CGTP_ERR_UNSUPPORTED
