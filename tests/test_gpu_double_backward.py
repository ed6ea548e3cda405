"""GPU parity of the double backward (cgtp_conv_bwd_bwd) against the oracle.

The oracle's double backward is pinned on the CPU by exact finite
differences of the backward; here the HIP path is compared with it element
by element on seeded inputs: every lane geometry and channel-count class,
mixed degrees, path-weight sharing, missing cotangents, results left out,
a grid many rounds of blocks deep and empty graphs.
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
        degs[[0, 5, 6, 33]] = 0      # receivers without in-edges
        degs[8] = N - 1              # the longest possible segment
        degs[9] = 17                 # not a multiple of the edges in flight per wave
    return synth.random_graph(N, degs, seed=seed + 1)


def _inputs(rng, N, E, li, ls, lo, C, rows):
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    return dict(x=f(N, (li + 1) ** 2, C), W=f(E, rows, C), G=f(N, (lo + 1) ** 2, C),
                ggx=f(N, (li + 1) ** 2, C), ggY=f(E, (ls + 1) ** 2), ggW=f(E, rows, C))


def run_dbl(torch, dev, oracle, li, ls, lo, C, N=70, seed=0, shared=False, drop=(), want=("x", "Y", "W", "grad_out"),
            max_deg=12):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    g = _graph(N, seed=li * 1000 + ls * 100 + lo * 10 + C + seed, max_deg=max_deg)
    E = g.n_edges
    plan = Plan(li, ls, lo, C, shared_weights=shared)
    rng = np.random.default_rng(seed + 17)
    a = _inputs(rng, N, E, li, ls, lo, C, plan.weight_rows)
    Y = oracle.sh(ls, g.r).astype(np.float32)
    for k in drop:
        a[k] = None
    _log(f"[dbl] ({li},{ls},{lo}) C={C} N={N} E={E} shared={shared} drop={drop} want={want}")
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev) if v is not None else None
    rp, sr = T(g.row_ptr), T(g.src)
    got = plan.conv_bwd_bwd(rp, sr, T(a["x"]), T(Y), T(a["W"]), T(a["G"]), T(a["ggx"]), T(a["ggY"]),
                            T(a["ggW"]), want=want)
    got = [t.cpu().numpy() if t is not None else None for t in got]
    if shared:
        ref = oracle.conv_bwd_bwd_shared(li, ls, lo, g.row_ptr, g.src, a["x"], Y, a["W"][:, 0], a["G"], a["ggx"],
                                         a["ggY"], a["ggW"][:, 0] if a["ggW"] is not None else None)
        ref = (ref[0], ref[1], ref[2][:, None, :], ref[3])
    else:
        ref = oracle.conv_bwd_bwd(li, ls, lo, g.row_ptr, g.src, a["x"], Y, a["W"], a["G"], a["ggx"], a["ggY"],
                                  a["ggW"])
    for name, key, u, v in zip(("dd_x", "dd_Y", "dd_W", "dd_out"), ("x", "Y", "W", "grad_out"), got, ref):
        if key not in want:
            assert u is None
            continue
        assert_parity(u, v, name)
    return g, got


CHANNELS = (1, 8, 12, 16, 32, 40, 64, 96, 128)


@pytest.mark.parametrize("L,C", [(L, C) for L in (1, 2, 3) for C in CHANNELS])
def test_double_backward_every_geometry(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    g, (dx, dY, dW, dout) = run_dbl(torch, dev, oracle, L, L, L, C)
    # a receiver without in-edges gets zeros in dd_out, a sender without out-edges in dd_x
    assert np.all(dout[[0, 5, 6, 33]] == 0)
    no_out = np.setdiff1d(np.arange(g.n_nodes), g.src)
    assert np.all(dx[no_out] == 0)


@pytest.mark.parametrize("li,ls,lo,C", [(2, 1, 3, 24), (3, 2, 1, 24), (1, 3, 2, 96), (0, 1, 1, 16), (2, 2, 0, 8),
                                        (3, 3, 2, 128), (1, 0, 1, 40), (0, 0, 0, 64), (3, 2, 1, 64), (2, 3, 3, 48)])
def test_double_backward_mixed_degrees(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_dbl(torch, dev, oracle, li, ls, lo, C)


@pytest.mark.parametrize("li,ls,lo,C", [(1, 1, 1, 8), (2, 2, 2, 128), (2, 3, 2, 96), (3, 3, 3, 64)])
def test_double_backward_shared_path_weights(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_dbl(torch, dev, oracle, li, ls, lo, C, shared=True)


@pytest.mark.parametrize("drop", [("ggx",), ("ggY",), ("ggW",), ("ggx", "ggW"), ("ggx", "ggY", "ggW")])
def test_double_backward_missing_cotangents(torch_dev, oracle, drop):
    """A cotangent passed as NULL counts as zero (all three NULL: zero results)."""
    torch, dev = torch_dev
    for L, C in ((2, 32), (3, 128), (3, 64)):
        _, got = run_dbl(torch, dev, oracle, L, L, L, C, drop=drop)
        if len(drop) == 3:
            assert all(np.count_nonzero(t) == 0 for t in got)


@pytest.mark.parametrize("want", [("grad_out",), ("x",), ("Y", "W"), ("x", "W")])
@pytest.mark.parametrize("L", [2, 3])
def test_double_backward_partial_results(torch_dev, oracle, want, L):
    torch, dev = torch_dev
    run_dbl(torch, dev, oracle, L, L, L, 64, want=want)


@pytest.mark.parametrize("L,C", [(1, 128), (2, 64), (3, 16), (3, 48)])
def test_double_backward_many_nodes(torch_dev, oracle, L, C):
    """A grid many rounds of resident blocks deep with short ragged segments."""
    torch, dev = torch_dev
    run_dbl(torch, dev, oracle, L, L, L, C, N=5003, max_deg=7)


def test_double_backward_empty_graph(torch_dev):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64)
    for N in (9, 1):
        rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        sr = torch.zeros(0, dtype=torch.int32, device=dev)
        x = torch.randn(N, 9, 64, device=dev)
        G = torch.randn(N, 9, 64, device=dev)
        Y = torch.zeros(0, 9, device=dev)
        W = torch.zeros(0, 15, 64, device=dev)
        dx, dY, dW, dout = plan.conv_bwd_bwd(rp, sr, x, Y, W, G, torch.randn_like(x), Y, W)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dx) == 0 and torch.count_nonzero(dout) == 0
        assert dW.shape == (0, 15, 64) and dY.shape == (0, 9)
