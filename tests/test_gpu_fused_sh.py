"""GPU parity of the convolution with the spherical harmonics evaluated inside
the kernels (cgtp_conv_fwd_sh / cgtp_conv_bwd_sh) against the oracle.

The reference is the oracle's convolution with Y = the oracle's fp64 SH of the
same fp32 edge vectors (the fused kernels do not round Y to fp32 either), and
for the backward the oracle's SH backward applied to the oracle's grad_Y.  The
oracle's SH and SH backward are pinned on the CPU (scipy's complex harmonics,
the addition theorem, central differences).

Cases: every lane geometry (C = 8 and 24: several edges per wave; 64: one
slice per edge; 100 and 128: two slices per edge), every degree up to 3, mixed
degrees and path-weight sharing (the SUB form), a grid many rounds of blocks
deep, the 2000-atom layer, an empty graph, repeat runs (bitwise equal).  The
fused results also agree with the unfused chain (SH kernel, convolution, SH
backward) to the fp32 rounding of Y.
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
    degs = np.minimum(rng.integers(0, max_deg, size=N), N - 1)
    if N > 40:
        degs[[0, 5, 6, 33]] = 0
        degs[8] = N - 1
        degs[9] = 17
    return synth.random_graph(N, degs, seed=seed + 1)


def _reference(oracle, li, ls, lo, g, x, W, G, shared, P):
    Y64 = oracle.sh(ls, g.r)
    Wfull = np.repeat(W, P, axis=1) if shared else W
    ro = oracle.conv_fwd(li, ls, lo, g.row_ptr, g.src, x, Y64, Wfull)
    rdx, rdW, rdY = oracle.conv_bwd(li, ls, lo, g.row_ptr, g.src, x, Y64, Wfull, G)
    if shared:
        rdW = rdW.sum(axis=1, keepdims=True)
    return ro, rdx, rdW, oracle.sh_bwd(ls, g.r, rdY)


def run_fused(torch, dev, oracle, li, ls, lo, C, N=70, seed=0, shared=False, max_deg=12, g=None):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    if g is None:
        g = _graph(N, seed=li * 1000 + ls * 100 + lo * 10 + C + seed, max_deg=max_deg)
    N, E = g.n_nodes, g.n_edges
    plan = Plan(li, ls, lo, C, shared_weights=shared)
    rng = np.random.default_rng(seed + 11)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x, W, G = f(N, plan.dim_in, C), f(E, plan.weight_rows, C), f(N, plan.dim_out, C)
    _log(f"[fused-sh] ({li},{ls},{lo}) C={C} N={N} E={E} shared={shared}")
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rp, sr, r = T(g.row_ptr), T(g.src), T(g.r)
    ws = plan.graph_prepare(rp, sr)
    out = plan.conv_fwd_sh(rp, sr, T(x), r, T(W), ws).cpu().numpy()
    dx, dW, dr = (t.cpu().numpy() for t in plan.conv_bwd_sh(rp, sr, T(x), r, T(W), T(G), ws))
    ro, rdx, rdW, rdr = _reference(oracle, li, ls, lo, g, x, W, G, shared, len(plan.paths))
    assert_parity(out, ro, "out")
    assert_parity(dx, rdx, "dx")
    assert_parity(dW, rdW, "dW")
    if ls == 0:
        assert np.all(dr == 0)  # a constant harmonic has no gradient
    else:
        assert_parity(dr, rdr, "grad_r")
    return g, plan, out, dx, dW, dr


CHANNELS = (8, 24, 64, 100, 128)


@pytest.mark.parametrize("L,C", [(L, C) for L in (1, 2, 3) for C in CHANNELS])
def test_fused_sh_every_geometry(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    run_fused(torch, dev, oracle, L, L, L, C)


@pytest.mark.parametrize("li,ls,lo,C", [(2, 1, 3, 24), (3, 2, 1, 64), (1, 3, 2, 96), (0, 1, 1, 16), (2, 2, 0, 8),
                                        (3, 3, 2, 128), (1, 0, 1, 32), (2, 2, 1, 48)])
def test_fused_sh_mixed_degrees(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_fused(torch, dev, oracle, li, ls, lo, C)


@pytest.mark.parametrize("li,ls,lo,C", [(2, 2, 2, 128), (3, 3, 3, 64), (1, 2, 2, 16), (2, 2, 2, 40)])
def test_fused_sh_shared_weights(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_fused(torch, dev, oracle, li, ls, lo, C, shared=True)


@pytest.mark.parametrize("L,C", [(2, 128), (2, 24), (3, 64)])
def test_fused_sh_many_nodes(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    run_fused(torch, dev, oracle, L, L, L, C, N=5003, max_deg=7)


def test_fused_sh_layer_and_unfused_chain(torch_dev, oracle):
    """The 2000-atom layer (L = 2, C = 128) against the oracle; the fused
    results against the unfused chain sh -> conv -> sh_bwd on the same
    inputs (they differ by the fp32 rounding of Y only); grad_r orthogonal to
    r (the harmonics depend on the direction only); repeat runs bitwise
    equal."""
    torch, dev = torch_dev
    w = synth.WORKLOADS["layer"]
    g = synth.make_graph(w)
    g_, plan, out, dx, dW, dr = run_fused(torch, dev, oracle, 2, 2, 2, 128, g=g, seed=3)
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rng = np.random.default_rng(3 + 11)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x, W, G = f(g.n_nodes, 9, 128), f(g.n_edges, 15, 128), f(g.n_nodes, 9, 128)
    rp, sr, r = T(g.row_ptr), T(g.src), T(g.r)
    Y = plan.sh(r)
    out_u = plan.conv_fwd(rp, sr, T(x), Y, T(W)).cpu().numpy()
    dx_u, dW_u, dY_u = plan.conv_bwd(rp, sr, T(x), Y, T(W), T(G))
    dr_u = plan.sh_bwd(r, dY_u).cpu().numpy()
    for a, b, n in ((out, out_u, "out"), (dx, dx_u.cpu().numpy(), "dx"), (dW, dW_u.cpu().numpy(), "dW"),
                    (dr, dr_u, "grad_r")):
        assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b), n
    rr = g.r.astype(np.float64)
    cos = np.abs(np.sum(dr * rr, axis=1)) / (np.linalg.norm(dr, axis=1) * np.linalg.norm(rr, axis=1) + 1e-30)
    assert np.max(cos) < 1e-4
    dx2, dW2, dr2 = (t.cpu().numpy() for t in plan.conv_bwd_sh(rp, sr, T(x), r, T(W), T(G)))
    out2 = plan.conv_fwd_sh(rp, sr, T(x), r, T(W)).cpu().numpy()
    assert np.array_equal(out2, out) and np.array_equal(dx2, dx) and np.array_equal(dW2, dW)
    assert np.array_equal(dr2, dr)


def test_fused_sh_empty_graph_and_optional_outputs(torch_dev, oracle):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64)
    N = 9
    rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    sr = torch.zeros(0, dtype=torch.int32, device=dev)
    x = torch.randn(N, 9, 64, device=dev)
    r = torch.zeros(0, 3, device=dev)
    W = torch.zeros(0, 15, 64, device=dev)
    out = plan.conv_fwd_sh(rp, sr, x, r, W)
    dx, dW, dr = plan.conv_bwd_sh(rp, sr, x, r, W, torch.randn(N, 9, 64, device=dev))
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0 and torch.count_nonzero(dx) == 0 and dr.shape == (0, 3)
    # only grad_r requested, on a small graph
    g = _graph(70, seed=4)
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rng = np.random.default_rng(9)
    x, W, G = (rng.standard_normal(s, dtype=np.float32) for s in ((70, 9, 64), (g.n_edges, 15, 64), (70, 9, 64)))
    gx, gW, gr = plan.conv_bwd_sh(T(g.row_ptr), T(g.src), T(x), T(g.r), T(W), T(G), want=("dr",))
    assert gx is None and gW is None
    _, rdx, rdW, rdr = _reference(oracle, 2, 2, 2, g, x, W, G, False, 15)
    assert_parity(gr.cpu().numpy(), rdr, "grad_r alone")
    # grad_x and grad_W without grad_r
    gx, gW, gr = plan.conv_bwd_sh(T(g.row_ptr), T(g.src), T(x), T(g.r), T(W), T(G), want=("dx", "dW"))
    assert gr is None
    assert_parity(gx.cpu().numpy(), rdx, "grad_x without grad_r")
    assert_parity(gW.cpu().numpy(), rdW, "grad_W without grad_r")
