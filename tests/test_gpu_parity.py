"""GPU parity: libcgtp.so (through its C ABI) against the fp64 oracle.

Every workload's inputs come from the seeded generator; the oracle receives
exact copies of what the GPU received.  The convolution is fed the oracle's
spherical harmonics rounded to fp32 (the SH kernel is checked on its own), so
both sides see the same Y.

Every one of the five workloads is compared over its whole output tensors
(out, grad_x, grad_W, grad_Y): the small ones in one oracle call, the large
ones in chunks (receiver ranges for out, sender ranges for grad_x, edge
ranges for grad_W and grad_Y) whose squared errors and elementwise relative
errors are accumulated over the whole tensor (tests/metrics.py,
WholeTensor).  Edge cases cover every lane geometry and channel count
class, every degree triple up to 3, ragged and empty segments, hub senders
and many rounds of resident blocks.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import synth
from tests.layout import ws_sections
from tests.metrics import WholeTensor, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _log(*a):
    print(*a, flush=True)


def recv_of(row_ptr):
    return np.repeat(np.arange(row_ptr.shape[0] - 1), np.diff(row_ptr))


class Run:
    """A workload run on the GPU: inputs and all outputs, kept on the device."""

    def __init__(self, torch, dev, key, oracle, seed=0):
        w = synth.WORKLOADS[key]
        from clebsch_gordan_tensor_cgtp_amd.ops import Plan
        self.w, self.torch, self.dev = w, torch, dev
        g = synth.make_graph(w, seed)
        self.g = g
        N, E, L, C = g.n_nodes, g.n_edges, w.l_max, w.channels
        _log(f"[run] {key}: N={N} E={E} L={L} C={C}")
        self.plan = Plan(L, L, L, C)
        self.row_ptr = torch.from_numpy(g.row_ptr).to(dev)
        self.src = torch.from_numpy(g.src).to(dev)
        if E * w.num_paths * C <= 400_000_000:
            x, W, G = synth.make_tensors_numpy(N, E, L, C, seed)
            self.x, self.W, self.G = (torch.from_numpy(a).to(dev) for a in (x, W, G))
        else:
            self.x, self.W, self.G = synth.make_tensors_torch(N, E, L, C, dev, seed)
        # Y fed to the convolution: oracle SH of the same fp32 vectors, rounded to fp32
        self.Y = torch.from_numpy(oracle.sh(L, g.r).astype(np.float32)).to(dev)
        self.ws = self.plan.graph_prepare(self.row_ptr, self.src)
        self.out = self.plan.conv_fwd(self.row_ptr, self.src, self.x, self.Y, self.W, self.ws)
        self.dx, self.dW, self.dY = self.plan.conv_bwd(self.row_ptr, self.src, self.x, self.Y, self.W,
                                                      self.G, self.ws)
        torch.cuda.synchronize()

    def host(self, t, idx=None):
        if idx is not None:
            t = t[self.torch.as_tensor(np.asarray(idx), device=t.device, dtype=self.torch.int64)]
        return t.cpu().numpy()


_RUNS = {}


def get_run(torch_dev, key, oracle):
    if key not in _RUNS:
        torch, dev = torch_dev
        _RUNS.clear()
        torch.cuda.empty_cache()
        _RUNS[key] = Run(torch, dev, key, oracle)
    return _RUNS[key]


def _chunks(bounds, limit):
    """Split [0, n) into ranges [a, b) of consecutive items whose weight
    (bounds[b] - bounds[a]) stays near `limit` (at least one item each)."""
    n = bounds.shape[0] - 1
    a = 0
    while a < n:
        b = int(np.searchsorted(bounds, bounds[a] + limit, side="right")) - 1
        b = max(b, a + 1)
        b = min(b, n)
        yield a, b
        a = b


# ---------------------------------------------------------------------------
# spherical harmonics and graph preparation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["tiny", "layer", "high_l", "dense", "large"])
def test_sh_parity(torch_dev, oracle, key):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    w = synth.WORKLOADS[key]
    g = synth.make_graph(w)
    _log(f"[sh] {key}: E={g.n_edges} L={w.l_max}")
    plan = Plan(w.l_max, w.l_max, w.l_max, w.channels)
    Y = plan.sh(torch.from_numpy(g.r).to(dev)).cpu().numpy()
    assert_parity(Y, oracle.sh(w.l_max, g.r), f"Y[{key}]")


@pytest.mark.parametrize("l_sh", [0, 1, 2, 3])
def test_sh_every_degree(torch_dev, oracle, l_sh):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    r = np.random.default_rng(l_sh).normal(size=(1000, 3)).astype(np.float32)
    Y = Plan(1, l_sh, 1, 8).sh(torch.from_numpy(r).to(dev)).cpu().numpy()
    assert_parity(Y, oracle.sh(l_sh, r), f"Y[l_sh={l_sh}]")


def read_view(ws, N, E):
    s = ws_sections(N, E)
    iv = lambda name, n: ws[s[name]:s[name] + 4 * n].view(np.int32)
    return {k: iv(k, n) for k, n in (("srow", N + 1), ("perm", E), ("sdst", E), ("center", N),
                                     ("rorder", s["grid"]), ("sorder", s["grid"]))}


def check_schedule(order, deg, N, name, locality):
    """A block schedule over 8*ceil(N/8) blocks; every node exactly once.
    Default: all nodes longest first, then idle blocks.  Locality: range x
    (blocks x, x+8, ...) holds n_x = clamp(N - xQ, 0, Q) nodes, longest first,
    then idle blocks."""
    assert order.shape[0] == 8 * ((N + 7) // 8)
    got = order[order >= 0]
    np.testing.assert_array_equal(np.sort(got), np.arange(N), err_msg=name)
    assert np.all(order[order < 0] == -1)
    d = np.minimum(deg, 1023)
    if not locality:
        assert np.all(order[:N] >= 0)
        assert np.all(np.diff(d[order[:N]]) <= 0), name
        return
    Q = (N + 7) // 8
    for x in range(8):
        part = order[x::8]
        nx = min(max(N - x * Q, 0), Q)
        assert np.all(part[:nx] >= 0) and np.all(part[nx:] == -1), (name, x)
        assert np.all(np.diff(d[part[:nx]]) <= 0), (name, x)


@pytest.mark.parametrize("key", ["tiny", "layer", "dense", "large"])
@pytest.mark.parametrize("locality", [True, False])
def test_graph_prepare(torch_dev, oracle, key, locality):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    w = synth.WORKLOADS[key]
    g = synth.make_graph(w)
    N, E = g.n_nodes, g.n_edges
    _log(f"[prep] {key}: N={N} E={E} locality={locality}")
    plan = Plan(w.l_max, w.l_max, w.l_max, w.channels, locality=locality)
    ws = plan.graph_prepare(torch.from_numpy(g.row_ptr).to(dev), torch.from_numpy(g.src).to(dev)).cpu().numpy()
    v = read_view(ws, N, E)
    # the sender-sorted view is the stable counting sort of the edges by sender
    rs, rp, rd = oracle.graph_transpose(g.row_ptr, g.src)
    np.testing.assert_array_equal(v["srow"], rs)
    np.testing.assert_array_equal(v["perm"], rp)
    np.testing.assert_array_equal(v["sdst"], rd)
    check_schedule(v["rorder"], np.diff(g.row_ptr), N, "rorder", locality)
    check_schedule(v["sorder"], np.diff(rs), N, "sorder", locality)
    if locality:
        xcd_of = np.empty(N, np.int64)
        for x in range(8):
            part = v["rorder"][x::8]
            xcd_of[part[part >= 0]] = x
        # clusters: every centre is a valid node, and each cluster's members
        # occupy consecutive ranges
        c = v["center"]
        assert np.all((c >= 0) & (c < N))
        for cc in np.unique(c):
            xs = np.unique(xcd_of[c == cc])
            assert xs.max() - xs.min() + 1 == xs.shape[0], cc


@pytest.mark.parametrize("N", [1, 7, 1023, 1024, 1025, 2049, 3073])
def test_graph_prepare_block_boundaries(torch_dev, oracle, N):
    """The longest-first schedules are built 1024 nodes per block: node counts
    at and around the block size, a last block with one node, nodes with no
    in- or out-edges, degrees from 0 to 40."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(N)
    degs = np.minimum(rng.integers(0, 41, size=N), N - 1)
    degs[rng.random(N) < 0.1] = 0
    g = synth.random_graph(N, degs, seed=N + 3)
    E = g.n_edges
    _log(f"[prep-blocks] N={N} E={E}")
    plan = Plan(1, 1, 1, 8)
    ws = plan.graph_prepare(torch.from_numpy(g.row_ptr).to(dev), torch.from_numpy(g.src).to(dev)).cpu().numpy()
    v = read_view(ws, N, E)
    rs, rp, rd = oracle.graph_transpose(g.row_ptr, g.src)
    np.testing.assert_array_equal(v["srow"], rs)
    np.testing.assert_array_equal(v["perm"], rp)
    np.testing.assert_array_equal(v["sdst"], rd)
    check_schedule(v["rorder"], np.diff(g.row_ptr), N, "rorder", False)
    check_schedule(v["sorder"], np.diff(rs), N, "sorder", False)


def test_graph_prepare_hub_sender(torch_dev, oracle):
    """One sender with about 3000 out-edges (ranked chunk by chunk) and one
    with 1500, inside an otherwise sparse random graph."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(5)
    N = 3200
    recv, send = [], []
    for i in range(N):
        nb = set(rng.choice(N, size=rng.integers(0, 6), replace=False).tolist())
        if i != 0:
            nb.add(0)                      # hub 0 sends to every other node
        if i != 1 and i % 2 == 0:
            nb.add(1)                      # node 1 to every second node
        nb.discard(i)
        for j in sorted(nb):
            recv.append(i)
            send.append(j)
    recv, send = np.array(recv), np.array(send)
    row_ptr = np.zeros(N + 1, np.int64)
    np.cumsum(np.bincount(recv, minlength=N), out=row_ptr[1:])
    E = send.shape[0]
    _log(f"[hub] N={N} E={E} out-degree of node 0: {(send == 0).sum()}")
    plan = Plan(1, 1, 1, 16)
    rp_d = torch.from_numpy(row_ptr.astype(np.int32)).to(dev)
    src_d = torch.from_numpy(send.astype(np.int32)).to(dev)
    ws = plan.graph_prepare(rp_d, src_d)
    v = read_view(ws.cpu().numpy(), N, E)
    rs, rp, rd = oracle.graph_transpose(row_ptr, send)
    np.testing.assert_array_equal(v["srow"], rs)
    np.testing.assert_array_equal(v["perm"], rp)
    np.testing.assert_array_equal(v["sdst"], rd)
    # and the backward over it
    x, W, G = synth.make_tensors_numpy(N, E, 1, 16, seed=8)
    r = rng.normal(size=(E, 3)).astype(np.float32)
    Y = oracle.sh(1, r).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp_d, src_d, T(x), T(Y), T(W), T(G), ws))
    rdx, rdW, rdY = oracle.conv_bwd(1, 1, 1, row_ptr, send, x, Y, W, G)
    assert_parity(dx, rdx, "dx[hub]")
    assert_parity(dW, rdW, "dW[hub]")
    assert_parity(dY, rdY, "dY[hub]")


# ---------------------------------------------------------------------------
# convolution: whole tensors of every workload
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["tiny", "layer"])
def test_conv_full_parity(torch_dev, oracle, key):
    run = get_run(torch_dev, key, oracle)
    g, L = run.g, run.w.l_max
    x, W, G, Y = (run.host(t) for t in (run.x, run.W, run.G, run.Y))
    _log(f"[oracle] {key} fwd")
    out = oracle.conv_fwd(L, L, L, g.row_ptr, g.src, x, Y, W)
    assert_parity(run.host(run.out), out, f"out[{key}]")
    _log(f"[oracle] {key} bwd")
    dx, dW, dY = oracle.conv_bwd(L, L, L, g.row_ptr, g.src, x, Y, W, G)
    assert_parity(run.host(run.dx), dx, f"dx[{key}]")
    assert_parity(run.host(run.dW), dW, f"dW[{key}]")
    assert_parity(run.host(run.dY), dY, f"dY[{key}]")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["dense", "high_l", "large"])
def test_conv_whole_tensor_parity_chunked(torch_dev, oracle, key):
    """out, grad_x, grad_W and grad_Y of a large workload against the oracle,
    every entry of every tensor, in chunks that bound host memory."""
    torch, dev = torch_dev
    run = get_run(torch_dev, key, oracle)
    g, L = run.g, run.w.l_max
    N, E = g.n_nodes, g.n_edges
    rp = g.row_ptr.astype(np.int64)
    src = g.src.astype(np.int64)
    x64 = run.host(run.x).astype(np.float64)
    G64 = run.host(run.G).astype(np.float64)
    row_elems = run.plan.num_paths * run.plan.channels
    limit = max(1, (48 << 20) // row_elems)      # edges per chunk: about 48M weight entries

    def local_csr(e0, e1):
        return np.clip(rp - e0, 0, e1 - e0)

    # forward: receiver ranges
    acc = WholeTensor(torch, run.out, f"out[{key}]")
    for i0, i1 in _chunks(rp, limit):
        e0, e1 = int(rp[i0]), int(rp[i1])
        _log(f"[whole] {key} out receivers {i0}:{i1}")
        ref = oracle.conv_fwd(L, L, L, local_csr(e0, e1), src[e0:e1], x64, run.host(run.Y[e0:e1]),
                              run.host(run.W[e0:e1]))
        acc.add(run.out[i0:i1], ref[i0:i1])
    acc.check()

    # grad_W, grad_Y: edge ranges
    accW = WholeTensor(torch, run.dW, f"dW[{key}]")
    accY = WholeTensor(torch, run.dY, f"dY[{key}]")
    for e0 in range(0, E, limit):
        e1 = min(E, e0 + limit)
        _log(f"[whole] {key} dW/dY edges {e0}:{e1}")
        _, rdW, rdY = oracle.conv_bwd(L, L, L, local_csr(e0, e1), src[e0:e1], x64, run.host(run.Y[e0:e1]),
                                      run.host(run.W[e0:e1]), G64, want=("dW", "dY"))
        accW.add(run.dW[e0:e1], rdW)
        accY.add(run.dY[e0:e1], rdY)
    accW.check()
    accY.check()

    # grad_x: sender ranges, each with all of its out-edges
    srow, perm, sdst = oracle.graph_transpose(rp, src)
    accX = WholeTensor(torch, run.dx, f"dx[{key}]")
    for j0, j1 in _chunks(srow, max(limit, E // 8)):
        edges = perm[srow[j0]:srow[j1]]
        recv = sdst[srow[j0]:srow[j1]]
        order = np.lexsort((edges, recv))
        es = edges[order]
        lrp = np.zeros(N + 1, np.int64)
        np.cumsum(np.bincount(recv, minlength=N), out=lrp[1:])
        _log(f"[whole] {key} dx senders {j0}:{j1} ({es.shape[0]} edges)")
        rdx, _, _ = oracle.conv_bwd(L, L, L, lrp, src[es], x64, run.host(run.Y, es), run.host(run.W, es), G64,
                                    want=("dx",))
        accX.add(run.dx[j0:j1], rdx[j0:j1])
    accX.check()

    # the trilinear identity over the whole tensors (fp64 sums)
    Lval = acc.dot(run.G, run.out)
    scale = acc.norm(run.G) * acc.norm(run.out)
    for name, t, u in (("dx", run.dx, run.x), ("dW", run.dW, run.W), ("dY", run.dY, run.Y)):
        assert abs(acc.dot(t, u) - Lval) <= 1e-6 * scale, (key, name)


@pytest.mark.parametrize("key", ["layer", "high_l"])
def test_conv_deterministic(torch_dev, oracle, key):
    """Bitwise equal results from repeated calls and from a re-prepared
    graph (whose block placement may differ); high_l runs the degree-3
    backward whose two waves per edge split the paths."""
    torch, dev = torch_dev
    run = get_run(torch_dev, key, oracle)
    for k in range(3):
        ws = run.plan.graph_prepare(run.row_ptr, run.src) if k else run.ws
        out = run.plan.conv_fwd(run.row_ptr, run.src, run.x, run.Y, run.W, ws)
        dx, dW, dY = run.plan.conv_bwd(run.row_ptr, run.src, run.x, run.Y, run.W, run.G, ws)
        assert torch.equal(out, run.out)
        assert torch.equal(dx, run.dx) and torch.equal(dW, run.dW) and torch.equal(dY, run.dY)


@pytest.mark.parametrize("key", ["layer", "high_l"])
def test_optional_gradients(torch_dev, oracle, key):
    torch, dev = torch_dev
    run = get_run(torch_dev, key, oracle)
    args = (run.row_ptr, run.src, run.x, run.Y, run.W, run.G, run.ws)
    for want in (("dx",), ("dW",), ("dY",), ("dx", "dY"), ("dW", "dY"), ("dx", "dW")):
        got = run.plan.conv_bwd(*args, want=want)
        for name, full, part in zip(("dx", "dW", "dY"), (run.dx, run.dW, run.dY), got):
            if name in want:
                assert torch.equal(part, full), (want, name)
            else:
                assert part is None


# ---------------------------------------------------------------------------
# workspace handling
# ---------------------------------------------------------------------------
def _small_case(L, C, N=70, seed=0):
    rng = np.random.default_rng(seed)
    degs = rng.integers(0, 12, size=N)
    degs[[0, 5, 6, 33]] = 0
    degs[8] = N - 1
    g = synth.random_graph(N, degs, seed=seed + 1)
    return g


def test_unprepared_workspace_is_prepared_by_the_call(torch_dev, oracle):
    """A fresh (never prepared) workspace and a workspace prepared for another
    graph of the same size: the convolution prepares it itself."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    L, C = 2, 96
    plan = Plan(L, L, L, C)
    gA, gB = _small_case(L, C, seed=1), _small_case(L, C, seed=2)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dev_graph = {id(g): (T(g.row_ptr), T(g.src)) for g in (gA, gB)}   # distinct, live device arrays
    N = gA.n_nodes
    E = max(gA.n_edges, gB.n_edges)
    ws = torch.full((plan.workspace_size(N, E),), 0x7F, dtype=torch.uint8, device=dev)
    for g in (gA, gB, gA):
        x, W, G = synth.make_tensors_numpy(N, g.n_edges, L, C, seed=3)
        Y = oracle.sh(L, g.r).astype(np.float32)
        rp, sr = dev_graph[id(g)]
        out = plan.conv_fwd(rp, sr, T(x), T(Y), T(W), ws).cpu().numpy()
        dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G), ws))
        assert_parity(out, oracle.conv_fwd(L, L, L, g.row_ptr, g.src, x, Y, W), "out")
        rdx, rdW, rdY = oracle.conv_bwd(L, L, L, g.row_ptr, g.src, x, Y, W, G)
        assert_parity(dx, rdx, "dx")
        assert_parity(dW, rdW, "dW")
        assert_parity(dY, rdY, "dY")


def test_corrupt_view_stays_in_bounds(torch_dev, oracle):
    """A prepared workspace whose view is overwritten afterwards (sender
    offsets negative, huge or decreasing, edge and receiver ids out of range):
    the backward clamps every view index, returns normally, and the next
    properly prepared call is exact again."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    L, C = 1, 128
    plan = Plan(L, L, L, C)
    g = _small_case(L, C, seed=4)
    N, E = g.n_nodes, g.n_edges
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, W, G = synth.make_tensors_numpy(N, E, L, C, seed=5)
    Y = oracle.sh(L, g.r).astype(np.float32)
    rp, sr = T(g.row_ptr), T(g.src)
    ws = plan.graph_prepare(rp, sr)
    s = ws_sections(N, E)
    rng = np.random.default_rng(9)
    bad_srow = rng.choice(np.array([-(2 ** 31), -7, 0, 3, E // 2, E, E + 5, 2 ** 31 - 1], np.int64), size=N + 1)
    bad_perm = rng.choice(np.array([-1, 0, E - 1, E, 2 ** 31 - 1], np.int64), size=E)
    bad_sdst = rng.choice(np.array([-(2 ** 31), -1, 0, N - 1, N, 2 ** 30], np.int64), size=E)
    for name, arr in (("srow", bad_srow), ("perm", bad_perm), ("sdst", bad_sdst)):
        b = torch.from_numpy(arr.astype(np.int32).view(np.uint8)).to(dev)
        ws[s[name]:s[name] + b.numel()] = b
    outs = plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G), ws)   # the record still says "prepared"
    torch.cuda.synchronize()
    assert all(o is not None for o in outs)
    plan.graph_prepare(rp, sr, ws)
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G), ws))
    rdx, rdW, rdY = oracle.conv_bwd(L, L, L, g.row_ptr, g.src, x, Y, W, G)
    assert_parity(dx, rdx, "dx")
    assert_parity(dW, rdW, "dW")
    assert_parity(dY, rdY, "dY")


# ---------------------------------------------------------------------------
# edge cases: every lane geometry and channel count class, every degree
# triple, ragged and empty segments, many rounds of blocks, empty graphs
# ---------------------------------------------------------------------------
CHANNELS = (1, 3, 8, 12, 16, 24, 32, 40, 64, 72, 96, 128)
CASES = [(L, L, L, C) for L in (1, 2, 3) for C in CHANNELS]
TRIPLES = [(a, b, c) for a in range(4) for b in range(4) for c in range(4)]
MIXED = [(a, b, c, 24) for (a, b, c) in TRIPLES if not (a == b == c and a > 0)] + \
        [(a, b, c, 96) for (a, b, c) in ((0, 0, 0), (2, 3, 2), (3, 1, 2), (1, 3, 3), (3, 3, 0), (2, 2, 1))] + \
        [(2, 3, 2, 64), (3, 1, 2, 48), (1, 3, 3, 40), (0, 3, 3, 33)]  # degree 3, one 64-lane slice: path-split


def run_small(torch, dev, oracle, li, ls, lo, C, N=70, seed=0):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(li * 1000 + ls * 100 + lo * 10 + C)
    degs = rng.integers(0, 12, size=N)
    degs[[0, 5, 6, 33]] = 0          # receivers without in-edges
    degs[7] = 1
    degs[8] = N - 1                  # longest possible segment
    degs[9] = 17                     # not a multiple of the edges in flight per wave
    g = synth.random_graph(N, degs, seed=li * 100 + C + seed)
    x, W, G = synth.make_tensors_numpy(N, g.n_edges, max(li, ls, lo), C, seed=3, l_in=li, l_sh=ls, l_out=lo)
    Y = oracle.sh(ls, g.r).astype(np.float32)
    _log(f"[small] ({li},{ls},{lo}) C={C} N={N} E={g.n_edges}")
    plan = Plan(li, ls, lo, C)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    ws = plan.graph_prepare(rp, sr)
    out = plan.conv_fwd(rp, sr, T(x), T(Y), T(W), ws).cpu().numpy()
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G), ws))
    ro = oracle.conv_fwd(li, ls, lo, g.row_ptr, g.src, x, Y, W)
    rdx, rdW, rdY = oracle.conv_bwd(li, ls, lo, g.row_ptr, g.src, x, Y, W, G)
    assert_parity(out, ro, "out")
    assert_parity(dx, rdx, "dx")
    assert_parity(dW, rdW, "dW")
    assert_parity(dY, rdY, "dY")
    assert np.all(out[[0, 5, 6, 33]] == 0)
    no_out = np.setdiff1d(np.arange(N), g.src)
    assert np.all(dx[no_out] == 0)


@pytest.mark.parametrize("li,ls,lo,C", CASES)
def test_conv_ragged_small(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_small(torch, dev, oracle, li, ls, lo, C)


@pytest.mark.parametrize("li,ls,lo,C", MIXED)
def test_conv_mixed_degrees(torch_dev, oracle, li, ls, lo, C):
    torch, dev = torch_dev
    run_small(torch, dev, oracle, li, ls, lo, C)


@pytest.mark.parametrize("L,C", [(1, 8), (1, 128), (2, 16), (2, 64), (2, 100), (3, 40)])
def test_conv_many_nodes(torch_dev, oracle, L, C):
    """A grid many rounds of resident blocks deep, with short ragged segments
    and receivers without in-edges, for every lane mapping (C < 64, = 64,
    > 64), forward and backward."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(L * 77 + C)
    N = 5003
    degs = rng.integers(0, 7, size=N)
    g = synth.random_graph(N, degs, seed=L * 31 + C)
    x, W, G = synth.make_tensors_numpy(N, g.n_edges, L, C, seed=4)
    Y = oracle.sh(L, g.r).astype(np.float32)
    _log(f"[many nodes] L={L} C={C} N={N} E={g.n_edges}")
    plan = Plan(L, L, L, C)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    ws = plan.graph_prepare(rp, sr)
    out = plan.conv_fwd(rp, sr, T(x), T(Y), T(W), ws).cpu().numpy()
    assert_parity(out, oracle.conv_fwd(L, L, L, g.row_ptr, g.src, x, Y, W), "out")
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), T(W), T(G), ws))
    rdx, rdW, rdY = oracle.conv_bwd(L, L, L, g.row_ptr, g.src, x, Y, W, G)
    assert_parity(dx, rdx, "dx")
    assert_parity(dW, rdW, "dW")
    assert_parity(dY, rdY, "dY")


@pytest.mark.parametrize("L", [2, 3])  # 3: the path-split backward
def test_conv_empty_graph(torch_dev, oracle, L):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    C = 64
    plan = Plan(L, L, L, C)
    D, P = plan.dim_in, plan.num_paths
    for N in (9, 1):
        rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        sr = torch.zeros(0, dtype=torch.int32, device=dev)
        x = torch.randn(N, D, C, device=dev)
        Y = torch.zeros(0, D, device=dev)
        W = torch.zeros(0, P, C, device=dev)
        ws = plan.graph_prepare(rp, sr)
        out = plan.conv_fwd(rp, sr, x, Y, W, ws)
        dx, dW, dY = plan.conv_bwd(rp, sr, x, Y, W, torch.randn(N, D, C, device=dev), ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out) == 0 and torch.count_nonzero(dx) == 0
        assert dW.shape == (0, P, C) and dY.shape == (0, D)
    # no nodes at all
    rp0 = torch.zeros(1, dtype=torch.int32, device=dev)
    ws0 = plan.graph_prepare(rp0, sr)
    out0 = plan.conv_fwd(rp0, sr, torch.zeros(0, D, C, device=dev), Y, W, ws0)
    assert out0.shape == (0, D, C)
    assert plan.sh(torch.zeros(0, 3, device=dev)).shape == (0, D)


def test_validate_flag_rejects_malformed_csr(torch_dev):
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd import _lib
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(1, 1, 1, 8, validate=True)
    good_rp = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    src = torch.tensor([1, 0], dtype=torch.int32, device=dev)
    plan.graph_prepare(good_rp, src)
    for rp, s in (([0, 2, 1], [1, 0]), ([1, 1, 2], [1, 0]), ([0, 1, 3], [1, 0]), ([0, 1, 2], [1, 2]),
                  ([0, 1, 2], [-1, 0])):
        with pytest.raises(_lib.CgtpError) as ei:
            plan.graph_prepare(torch.tensor(rp, dtype=torch.int32, device=dev),
                               torch.tensor(s, dtype=torch.int32, device=dev))
        assert ei.value.status == _lib.CGTP_ERR_GRAPH


@pytest.mark.parametrize("li,ls,lo,C", [(1, 1, 1, 8), (2, 2, 2, 128), (2, 2, 2, 24), (3, 3, 3, 64), (2, 3, 2, 96),
                                        (1, 2, 2, 16), (3, 3, 3, 128)])
def test_conv_shared_path_weights(torch_dev, oracle, li, ls, lo, C):
    """Path-weight sharing: W and grad_W are [E][C] (one weight per edge and
    channel for every path); grad_W is the sum over the paths."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    N = 70
    rng = np.random.default_rng(li * 100 + ls * 10 + lo + C)
    degs = rng.integers(0, 12, size=N)
    degs[[0, 5]] = 0
    degs[8] = N - 1
    g = synth.random_graph(N, degs, seed=C + 5)
    E = g.n_edges
    x = rng.standard_normal((N, (li + 1) ** 2, C), dtype=np.float32)
    Ws = rng.standard_normal((E, C), dtype=np.float32)
    G = rng.standard_normal((N, (lo + 1) ** 2, C), dtype=np.float32)
    Y = oracle.sh(ls, g.r).astype(np.float32)
    _log(f"[shared] ({li},{ls},{lo}) C={C} N={N} E={E}")
    plan = Plan(li, ls, lo, C, shared_weights=True)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    Wd = T(Ws[:, None, :])                 # [E][1][C]: one weight row per edge
    out = plan.conv_fwd(rp, sr, T(x), T(Y), Wd).cpu().numpy()
    dx, dW, dY = (t.cpu().numpy() for t in plan.conv_bwd(rp, sr, T(x), T(Y), Wd, T(G)))
    assert dW.shape == (E, 1, C)
    assert_parity(out, oracle.conv_fwd_shared(li, ls, lo, g.row_ptr, g.src, x, Y, Ws), "out")
    rdx, rdW, rdY = oracle.conv_bwd_shared(li, ls, lo, g.row_ptr, g.src, x, Y, Ws, G)
    assert_parity(dx, rdx, "dx")
    assert_parity(dW[:, 0], rdW, "dW")
    assert_parity(dY, rdY, "dY")


def test_binding_prepares_the_workspaces_it_allocates(torch_dev, oracle):
    """A workspace freed after preparation and the same memory handed out
    again (torch's caching allocator returns the block at the same address)
    for other data: a call without ``ws`` must not take the library's record
    of that address for a prepared view."""
    torch, dev = torch_dev
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    L, C = 2, 64
    plan = Plan(L, L, L, C)
    g = _small_case(L, C, seed=6)
    N, E = g.n_nodes, g.n_edges
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rp, sr = T(g.row_ptr), T(g.src)
    x, W, G = synth.make_tensors_numpy(N, E, L, C, seed=7)
    Y = oracle.sh(L, g.r).astype(np.float32)
    ref = oracle.conv_fwd(L, L, L, g.row_ptr, g.src, x, Y, W)
    xd, Yd, Wd = T(x), T(Y), T(W)
    for _ in range(3):
        ws = plan.graph_prepare(rp, sr)
        nbytes = ws.numel()
        del ws
        junk = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev)   # likely the same block
        del junk
        out = plan.conv_fwd(rp, sr, xd, Yd, Wd).cpu().numpy()
        assert_parity(out, ref, "out")
