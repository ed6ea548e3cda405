"""GPU parity of the fully connected ("uvw") mixing of the per-path outputs
(cgtp_path_mix_fwd / cgtp_path_mix_bwd, fp64 matrix cores) against the
oracle, alone and composed with the per-path-output convolution into the
fully connected product.

The oracle's mixing is pinned on the CPU (identity matrices give the summed
convolution, diagonal ones the weight-scaled convolution; finite
differences).  Cases cover ragged node counts (partial 64-row tiles, a
partial last 32-node chunk, empty node-range splits), input and output
channel counts that are not multiples of the 32-deep chunks or the 64-wide
tiles or not of four (element loads instead of 16-byte loads), every degree
up to 3 and mixed degrees; operands that are not 16-byte aligned are
refused.
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


def run_mix(torch, dev, oracle, Ls, C, Co, N, seed=0):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(*Ls, C, path_outputs=True)
    rng = np.random.default_rng(seed + C + Co + N)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    mid, Wm, G = f(N, plan.mid_rows, C), f(plan.num_paths, C, Co), f(N, plan.dim_z, Co)
    _log(f"[mix] {Ls} C={C} C_out={Co} N={N}")
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    out = plan.path_mix_fwd(T(mid), T(Wm)).cpu().numpy()
    dmid, dW = (t.cpu().numpy() for t in plan.path_mix_bwd(T(mid), T(Wm), T(G)))
    assert_parity(out, oracle.path_mix_fwd(*Ls, mid, Wm), "out")
    rdm, rdW = oracle.path_mix_bwd(*Ls, mid, Wm, G)
    assert_parity(dmid, rdm, "d_mid")
    assert_parity(dW, rdW, "d_Wmix")


@pytest.mark.parametrize("Ls,C,Co,N", [((2, 2, 2), 128, 128, 2000), ((2, 2, 2), 64, 64, 70), ((1, 1, 1), 8, 8, 1),
                                       ((3, 3, 3), 64, 100, 333), ((2, 2, 2), 5, 7, 513), ((3, 3, 3), 16, 200, 1025),
                                       ((2, 1, 3), 24, 48, 96), ((0, 1, 1), 1, 1, 17), ((1, 2, 2), 128, 3, 4097),
                                       ((2, 2, 2), 36, 68, 2049), ((3, 2, 1), 96, 130, 95), ((2, 2, 2), 32, 40, 20001),
                                       ((1, 1, 1), 30, 64, 65)])
def test_path_mix(torch_dev, oracle, Ls, C, Co, N):
    torch, dev = torch_dev
    run_mix(torch, dev, oracle, Ls, C, Co, N)


@pytest.mark.parametrize("L,C,Co", [(2, 64, 128), (1, 16, 16), (3, 32, 64)])
def test_fully_connected_product_composed(torch_dev, oracle, L, C, Co):
    """The fully connected product on a graph: per-path-output convolution,
    then the mixing; forward and the chain of backwards, each call against the
    oracle on the inputs it received."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(L * 10 + C)
    N = 70
    degs = rng.integers(0, 12, size=N)
    g = synth.random_graph(N, degs, seed=L + C)
    plan = Plan(L, L, L, C, path_outputs=True)
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x, W, Wm = f(N, plan.dim_in, C), f(g.n_edges, plan.num_paths, C), f(plan.num_paths, C, Co)
    Gz = f(N, plan.dim_z, Co)
    Y = oracle.sh(L, g.r).astype(np.float32)
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    mid = plan.conv_fwd(rp, sr, T(x), T(Y), T(W))
    z = plan.path_mix_fwd(mid, T(Wm))
    gmid, gWm = plan.path_mix_bwd(mid, T(Wm), T(Gz))
    dx, dW, dY = plan.conv_bwd(rp, sr, T(x), T(Y), T(W), gmid)
    # each call against the oracle on the inputs it received (the per-path
    # outputs cross between the calls in fp32), and the whole chain within
    # the relative-L2 bound
    rmid = oracle.conv_fwd_mid(L, L, L, g.row_ptr, g.src, x, Y, W)
    mid_h = mid.cpu().numpy()
    assert_parity(mid_h, rmid, "mid")
    assert_parity(z.cpu().numpy(), oracle.path_mix_fwd(L, L, L, mid_h, Wm), "z")
    chain = oracle.path_mix_fwd(L, L, L, rmid, Wm)
    assert np.linalg.norm(z.cpu().numpy() - chain) <= 1e-5 * np.linalg.norm(chain)
    rgmid, rgWm = oracle.path_mix_bwd(L, L, L, mid_h, Wm, Gz)
    assert_parity(gmid.cpu().numpy(), rgmid, "d_mid")
    assert_parity(gWm.cpu().numpy(), rgWm, "d_Wmix")
    rdx, rdW, rdY = oracle.conv_bwd_mid(L, L, L, g.row_ptr, g.src, x, Y, W, gmid.cpu().numpy())
    assert_parity(dx.cpu().numpy(), rdx, "dx")
    assert_parity(dW.cpu().numpy(), rdW, "dW")
    assert_parity(dY.cpu().numpy(), rdY, "dY")


def test_path_mix_rejects_unaligned_operands(torch_dev):
    """The header requires 16-byte aligned arrays (the kernels load 16 bytes
    at a time): an operand 4 bytes into its allocation is refused."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd import _lib
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64, path_outputs=True)
    N = 30
    shape = (N, plan.mid_rows, 64)
    mid = torch.zeros(N * plan.mid_rows * 64 + 1, device=dev)[1:].view(shape)
    assert mid.data_ptr() % 16 == 4
    Wm = torch.randn(plan.num_paths, 64, 64, device=dev)
    with pytest.raises(_lib.CgtpError) as ei:
        plan.path_mix_fwd(mid, Wm)
    assert ei.value.status == _lib.CGTP_ERR_INVALID_ARG
    with pytest.raises(_lib.CgtpError) as ei:
        plan.path_mix_bwd(mid, Wm, torch.zeros(N, 9, 64, device=dev))
    assert ei.value.status == _lib.CGTP_ERR_INVALID_ARG


def test_path_mix_no_nodes(torch_dev):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 16, path_outputs=True)
    mid = torch.zeros(0, plan.mid_rows, 16, device=dev)
    Wm = torch.randn(plan.num_paths, 16, 8, device=dev)
    out = plan.path_mix_fwd(mid, Wm)
    gm, gw = plan.path_mix_bwd(mid, Wm, torch.zeros(0, 9, 8, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (0, 9, 8) and gm.shape == mid.shape
    assert torch.count_nonzero(gw) == 0
