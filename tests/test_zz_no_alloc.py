"""The allocation-free backward (cgtp_conv_bwd_noalloc, graph view in the
library's static device scratch) against the workspace backward
(cgtp_conv_bwd), called through the C ABI: two calls in a row, the second on
a smaller graph, each compared element by element (the two share their
kernels, so the results must be bitwise equal)."""
import ctypes

import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _case(torch, dev, oracle, N, L, C, seed):
    rng = np.random.default_rng(seed)
    g = synth.random_graph(N, rng.integers(0, 24, size=N), seed=seed)
    x, W, G = synth.make_tensors_numpy(N, g.n_edges, L, C, seed=seed + 1)
    Y = oracle.sh(L, g.r).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return g, T(g.row_ptr), T(g.src), T(x), T(Y), T(W), T(G)


@pytest.mark.parametrize("L,C", [(2, 128), (3, 64)])  # (3, 64): the path-split backward
def test_noalloc_backward_matches_workspace_backward(torch_dev, oracle, L, C):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd import _lib
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan, _ptr, _stream
    plan = Plan(L, L, L, C)
    lib = _lib.lib()
    for N, seed in ((3000, 11), (700, 12)):            # the second call is smaller
        g, rp, src, x, Y, W, G = _case(torch, dev, oracle, N, L, C, seed)
        E = g.n_edges
        print(f"[noalloc] L={L} C={C} N={N} E={E}", flush=True)
        ref = plan.conv_bwd(rp, src, x, Y, W, G)       # workspace path
        dx = torch.full((N, plan.dim_in, C), float("nan"), device=dev)
        dW = torch.full((E, plan.num_paths, C), float("nan"), device=dev)
        dY = torch.full((E, plan.dim_sh), float("nan"), device=dev)
        st = lib.cgtp_conv_bwd_noalloc(plan._h, N, E, _ptr(rp), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(G),
                                       _ptr(dx), _ptr(dW), _ptr(dY), _stream(dev))
        assert st == _lib.CGTP_OK, _lib.status_string(st)
        torch.cuda.synchronize()
        for name, got, want in (("dx", dx, ref[0]), ("dW", dW, ref[1]), ("dY", dY, ref[2])):
            assert torch.equal(got, want), (N, name)
    # the same graph again: the scratch already holds its view
    st = lib.cgtp_conv_bwd_noalloc(plan._h, N, E, _ptr(rp), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(G),
                                   _ptr(dx), _ptr(dW), _ptr(dY), _stream(dev))
    assert st == _lib.CGTP_OK
    torch.cuda.synchronize()
    assert torch.equal(dx, ref[0]) and torch.equal(dW, ref[1]) and torch.equal(dY, ref[2])
