"""The whole step (SH, graph preparation, forward, backward) captured in a HIP
graph and replayed.

The library's launch path makes no allocation, no memset and no host
synchronisation, so a caller can capture a step once and replay it, new
edge vectors, features and weights written into the same buffers before each
replay (the per-step loop of a simulation or of training on a fixed batch
shape).  Each replay is checked against an eager step on the same inputs,
with eager work and synchronisations between the replays; the kernels are
deterministic, so the results must be bitwise equal.
"""
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


@pytest.mark.parametrize("L,C,N", [(2, 128, 300), (1, 24, 200)])
def test_step_replayed_from_a_hip_graph(torch_dev, L, C, N):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(L * 100 + C)
    degs = rng.integers(0, 20, size=N)
    g = synth.random_graph(N, degs, seed=L + C)
    E = g.n_edges
    print(f"[graph] L={L} C={C} N={N} E={E}", flush=True)
    plan = Plan(L, L, L, C)
    T = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    rp, src = T(g.row_ptr), T(g.src)
    r, x = T(g.r), torch.randn(N, plan.dim_in, C, device=dev)
    W, G = torch.randn(E, plan.num_paths, C, device=dev), torch.randn(N, plan.dim_out, C, device=dev)
    Y = torch.empty(E, plan.dim_sh, device=dev)
    out = torch.empty(N, plan.dim_out, C, device=dev)
    dx, dW, dY = torch.empty_like(x), torch.empty_like(W), torch.empty_like(Y)
    ws = torch.empty(plan.workspace_size(N, E), dtype=torch.uint8, device=dev)

    def step():
        plan.sh(r, Y)
        plan.graph_prepare(rp, src, ws)
        plan.conv_fwd(rp, src, x, Y, W, ws, out=out)
        plan.conv_bwd(rp, src, x, Y, W, G, ws, grad_x=dx, grad_W=dW, grad_Y=dY)

    # warm up on a side stream, as capture requires, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for k in range(3):
        # new inputs in place, as a simulation or training loop writes them
        gen = torch.Generator(device=dev).manual_seed(k)
        r.add_(0.01 * torch.randn(r.shape, device=dev, generator=gen))  # stays clear of zero length
        x.copy_(torch.randn(x.shape, device=dev, generator=gen))
        W.copy_(torch.randn(W.shape, device=dev, generator=gen))
        G.copy_(torch.randn(G.shape, device=dev, generator=gen))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (Y, out, dx, dW, dY)]
        for t in (Y, out, dx, dW, dY):
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for a, b, name in zip(got, (Y, out, dx, dW, dY), ("Y", "out", "dx", "dW", "dY")):
            assert torch.equal(a, b), (k, name)
        assert torch.isfinite(out).all() and torch.isfinite(dx).all()
