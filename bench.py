"""Throughput of the CGTP convolution on one MI355X.

One step = one pass of the whole hot path over one synthetic layer: real
spherical harmonics of the edge vectors, graph preparation (sender-sorted
view and block schedules), forward convolution and backward convolution
(grad_x, grad_W, grad_Y).  The plan (paths and CG tables) is built once before
timing.  Inputs are resident in HBM before the timed region.  Prints one JSON
line on stdout; diagnostics go to stderr.

Headline workload (`value`): 2000 atoms at 0.1 atoms/A^3 with a 5 A cutoff
(about 106k directed edges), features, SH and outputs l = 0..2, C = 128, uvu
weights.  The same line carries the other single-GPU workloads under
"workloads": 50,000 atoms (L = 2, C = 128), 4,000 atoms with log-normal kNN
degrees 20-400 (L = 2, C = 128) and 10,000 atoms at L = 3, C = 64.

Other modes: --copy-ceiling (device copy rate), --copy-calibration (a plain
1 GiB copy for scaling HBM byte counters), --summarize DIR (turn the
rocprofv3 CSV output of the profile commands listed in profiles/ into the
summaries kept there), --cpu-single KEY (the oracle on one host thread; run
by the CPU baseline in a child process).
"""
import argparse
import csv
import hashlib
import json
import math
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6
KERNEL_SOURCES = ["clebsch_gordan_tensor_cgtp_amd/csrc/cgtp_kernels.h", "clebsch_gordan_tensor_cgtp_amd/csrc/cgtp_math.h",
                  "clebsch_gordan_tensor_cgtp_amd/csrc/cgtp_sh.h"]
HEADLINE = "layer"
OTHERS = ["large", "dense", "high_l"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(N, E, P, C, d_in, d_sh, d_out):
    """Bytes the method must move (each node row once; per-edge tensors once)."""
    fwd = E * (4 * P * C + 4 * d_sh + 4) + N * (4 * C * (d_in + d_out) + 4)
    bwd = E * (8 * P * C + 8 * d_sh + 8) + N * (4 * C * (2 * d_in + d_out) + 4)
    sh = E * (12 + 4 * d_sh)
    prep = E * 4 * 6 + N * 4 * 4
    # double backward: the receiver side reads W, ggW, Y, ggY per edge and
    # x, ggx per sender row and writes dd_out; the sender side reads W, ggW,
    # Y, ggY, the view and x, ggx, grad_out rows and writes dd_W, dd_Y, dd_x
    dbl_fwd = E * (8 * P * C + 8 * d_sh + 4) + N * (4 * C * (2 * d_in + d_out) + 4)
    dbl_bwd = E * (12 * P * C + 12 * d_sh + 8) + N * (4 * C * (3 * d_in + d_out) + 4)
    return {"fwd": fwd, "bwd": bwd, "sh": sh, "prep": prep, "dbl_fwd": dbl_fwd, "dbl_bwd": dbl_bwd}


def conv_flops(L, C, E):
    """fp64 flops per launch of the forward and the backward as the kernels
    execute them (fma = 2): forward q = x*y products, z = T q, acc += W z;
    backward R = T g, h = R y, v = R^T x, grad_x += W h, grad_W = x.h,
    grad_Y += W v -- counted from the real CG tables' nonzero pattern."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(L, L, L, 8)
    fwd = bwd = 0
    pairs_xy = set()
    for q, (l1, l2, l3) in enumerate(plan.paths):
        T = plan.export_cg(q)
        nz = T != 0
        fwd += 2 * int(nz.sum()) + 2 * (2 * l3 + 1)
        for a in range(2 * l1 + 1):
            for b in range(2 * l2 + 1):
                if nz[a, b].any():
                    pairs_xy.add((l1, a, l2, b))
        rab = int(nz.any(axis=2).sum())          # nonzero R[a][b]
        rows = int(nz.any(axis=(1, 2)).sum())     # a with any coefficient
        cols = int(nz.any(axis=(0, 2)).sum())     # b with any coefficient
        bwd += 2 * int(nz.sum()) + 4 * rab + 4 * rows + 2 * cols
    fwd += len(pairs_xy)                          # the shared x*y products
    return fwd * C * E, bwd * C * E


def read_summary(name):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def read_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch from a committed PMC summary, or None if
    absent or taken on other kernel sources."""
    kv = read_summary(f"pmc_{kernel}_{workload}.txt")
    if not kv or kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(torch, dev, key, seed=0):
    import numpy as np
    from clebsch_gordan_tensor_cgtp_amd import synth

    w = synth.WORKLOADS[key]
    g = synth.make_graph(w, seed)
    N, E, L, C = g.n_nodes, g.n_edges, w.l_max, w.channels
    if E * w.num_paths * C <= 400_000_000:
        x, W, G = (torch.from_numpy(a).to(dev) for a in synth.make_tensors_numpy(N, E, L, C, seed))
    else:
        x, W, G = synth.make_tensors_torch(N, E, L, C, dev, seed)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return w, g, T(g.row_ptr), T(g.src), T(g.r), x, W, G


def run_workload(torch, dev, key, steps, warmup, settle, locality=False, extras=True):
    """Time `steps` whole steps of workload `key`.  Returns the measurements
    and the host-side inputs (for the CPU baseline)."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan

    w, g, rp, src, r, x, W, G = make_inputs(torch, dev, key)
    N, E, L, C = g.n_nodes, g.n_edges, w.l_max, w.channels
    plan = Plan(L, L, L, C, locality=locality)
    P = plan.num_paths
    Y = torch.empty((E, plan.dim_sh), device=dev)
    out = torch.empty((N, plan.dim_out, C), device=dev)
    dx = torch.empty((N, plan.dim_in, C), device=dev)
    dW = torch.empty((E, P, C), device=dev)
    dY = torch.empty((E, plan.dim_sh), device=dev)
    ws = torch.empty(plan.workspace_size(N, E), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        plan.sh(r, Y)
        plan.graph_prepare(rp, src, ws)
        if ev:
            ev[1].record(stream)
        plan.conv_fwd(rp, src, x, Y, W, ws, out=out)
        if ev:
            ev[2].record(stream)
        plan.conv_bwd(rp, src, x, Y, W, G, ws, grad_x=dx, grad_W=dW, grad_Y=dY)
        if ev:
            ev[3].record(stream)

    log(f"workload {key}: N={N} E={E} L={L} C={C} P={P}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The GPU raises its clocks only after ~0.1-0.2 s of sustained load; keep
    # warming up (untimed) until the load has lasted `settle` seconds so the
    # timed steps see the loaded clock state a continuous training loop runs in.
    settle_steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(steps):
        step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = max(t_start.elapsed_time(t_end), wall * 1e3) / steps
    med = lambda a, b: statistics.median(e[a].elapsed_time(e[b]) for e in evs)
    prep_ms, fwd_ms, bwd_ms = med(0, 1), med(1, 2), med(2, 3)
    step_med = statistics.median(e[0].elapsed_time(e[3]) for e in evs)
    ab = algorithmic_bytes(N, E, P, C, plan.dim_in, plan.dim_sh, plan.dim_out)
    fl_fwd, fl_bwd = conv_flops(L, C, E)
    res = {
        "workload": w.name, "n_atoms": N, "n_edges": E, "l_max": L, "channels": C, "paths": P,
        "steps": steps, "settle_steps": settle_steps,
        "ms_per_step": ms_step, "ms_per_step_median": step_med,
        "edges_per_s": E / (ms_step * 1e-3),
        "sh_prep_ms": prep_ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_bwd_edges_per_s": E / ((fwd_ms + bwd_ms) * 1e-3),
        "fwd_alg_gbs": ab["fwd"] / (fwd_ms * 1e-3) / 1e9,
        "bwd_alg_gbs": ab["bwd"] / (bwd_ms * 1e-3) / 1e9,
        "fwd_hbm_frac": ab["fwd"] / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "bwd_hbm_frac": ab["bwd"] / (bwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "fwd_bwd_hbm_frac": (ab["fwd"] + ab["bwd"]) / ((fwd_ms + bwd_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "fwd_fp64_tflops": fl_fwd / (fwd_ms * 1e-3) / 1e12,
        "bwd_fp64_tflops": fl_bwd / (bwd_ms * 1e-3) / 1e12,
        "alg_bytes": {"fwd": ab["fwd"], "bwd": ab["bwd"]},
    }
    log(f"{key}: step {ms_step:.3f} ms | sh+prep {prep_ms:.3f} | fwd {fwd_ms:.3f} ms "
        f"({res['fwd_alg_gbs']:.0f} GB/s alg) | bwd {bwd_ms:.3f} ms ({res['bwd_alg_gbs']:.0f} GB/s alg)")
    if extras:
        res["forces"] = time_forces(torch, plan, stream, rp, src, r, Y, ws, steps)
        res["double_backward"] = time_double_backward(torch, plan, stream, rp, src, x, Y, W, G, ws, ab, steps)
        res["cp"] = time_cp(torch, plan, stream, rp, src, x, Y, G, (16, 32, 64) if key == HEADLINE else (32,),
                            steps)
        res["path_outputs"] = time_path_outputs(torch, stream, rp, src, x, Y, W, steps)
        res["fused_sh"] = time_fused_sh(torch, plan, stream, rp, src, x, r, Y, W, G, ws, ab, steps)
        res["graph_replay"] = time_graph_replay(torch, step, ms_step, steps)
    host = None
    if key == HEADLINE:
        host = (w, g, x.cpu().numpy(), W.cpu().numpy(), G.cpu().numpy())
    del Y, out, dx, dW, dY, ws, x, W, G
    torch.cuda.empty_cache()
    return res, host


def time_forces(torch, plan, stream, rp, src, r, Y, ws, steps):
    """Median launch times of the path from grad_Y to the forces: the SH
    backward (grad_Y -> grad_r) and the per-node gradient (grad_r ->
    grad_pos), HIP events on their stream.  Algorithmic bytes: r, grad_Y read
    and grad_r written per edge; grad_r and the view entry read per edge and
    grad_pos, row_ptr, srow per node."""
    N, E = rp.shape[0] - 1, r.shape[0]
    gY = torch.randn_like(Y)
    gr = torch.empty((E, 3), device=r.device)
    gp = torch.empty((N, 3), device=r.device)
    legs = {"sh_bwd": (lambda: plan.sh_bwd(r, gY, gr), E * (12 + 4 * plan.dim_sh + 12)),
            "node_grad": (lambda: plan.node_grad(rp, src, gr, ws, gp), E * (12 + 4) + N * (12 + 8))}
    res = {}
    for name, (fn, nbytes) in legs.items():
        for _ in range(3):
            fn()
        ts = []
        for _ in range(max(5, steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = statistics.median(a.elapsed_time(b) for a, b in ts)
        res[name] = {"ms": ms, "alg_bytes": nbytes, "alg_gbs": nbytes / (ms * 1e-3) / 1e9}
    log(f"  forces: sh_bwd {res['sh_bwd']['ms'] * 1e3:.1f} us | node_grad {res['node_grad']['ms'] * 1e3:.1f} us")
    return res


def time_graph_replay(torch, step, ms_step, steps):
    """The same step captured once in a HIP graph and replayed (the inputs
    stay in place): ms per step over `steps` replays, HIP events on the
    current stream, beside the eager launches' figure."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    res = {"ms_per_step": e0.elapsed_time(e1) / steps, "eager_ms_per_step": ms_step}
    log(f"  graph replay: {res['ms_per_step']:.3f} ms per step (eager launches {ms_step:.3f} ms)")
    del graph
    return res


def time_fused_sh(torch, plan, stream, rp, src, x, r, Y, W, G, ws, ab, steps):
    """The convolution with the SH evaluated in the kernels: median launch
    times of conv_fwd_sh and conv_bwd_sh (grad_x, grad_W, grad_r), and of the
    two chains from edge vectors to grad_r (graph already prepared): unfused
    sh -> conv_fwd -> conv_bwd -> sh_bwd, fused conv_fwd_sh -> conv_bwd_sh.
    Algorithmic bytes: the plain kernels' with Y (4 (l_sh+1)^2 bytes per edge)
    read as r (12 bytes), and grad_Y written as grad_r (12 bytes)."""
    E, dsh = r.shape[0], plan.dim_sh
    out = torch.empty((x.shape[0], plan.dim_out, x.shape[2]), device=x.device)
    fwd_b = ab["fwd"] - E * 4 * dsh + E * 12
    bwd_b = ab["bwd"] - E * 8 * dsh + E * 24

    def unfused():
        Yc = plan.sh(r)
        plan.conv_fwd(rp, src, x, Yc, W, ws, out=out)
        _, _, dYc = plan.conv_bwd(rp, src, x, Yc, W, G, ws)
        plan.sh_bwd(r, dYc)

    def fused():
        plan.conv_fwd_sh(rp, src, x, r, W, ws, out=out)
        plan.conv_bwd_sh(rp, src, x, r, W, G, ws)

    res = {"fwd_sh_ms": _median_ms(torch, stream, lambda: plan.conv_fwd_sh(rp, src, x, r, W, ws, out=out), steps),
           "bwd_sh_ms": _median_ms(torch, stream, lambda: plan.conv_bwd_sh(rp, src, x, r, W, G, ws), steps),
           "chain_unfused_ms": _median_ms(torch, stream, unfused, steps),
           "chain_fused_ms": _median_ms(torch, stream, fused, steps)}
    res["fwd_sh_alg_gbs"] = fwd_b / (res["fwd_sh_ms"] * 1e-3) / 1e9
    res["bwd_sh_alg_gbs"] = bwd_b / (res["bwd_sh_ms"] * 1e-3) / 1e9
    res["alg_bytes"] = {"fwd_sh": fwd_b, "bwd_sh": bwd_b}
    log(f"  fused SH: fwd {res['fwd_sh_ms']:.3f} ms ({res['fwd_sh_alg_gbs']:.0f} GB/s alg) | bwd "
        f"{res['bwd_sh_ms']:.3f} ms ({res['bwd_sh_alg_gbs']:.0f} GB/s alg) | r -> grad_r chain: unfused "
        f"{res['chain_unfused_ms']:.3f} ms, fused {res['chain_fused_ms']:.3f} ms")
    del out
    return res


def time_double_backward(torch, plan, stream, rp, src, x, Y, W, G, ws, ab, steps):
    """Median launch times of the double backward's two kernels (all three
    cotangents given): the receiver side (dd_out) and the sender side
    (dd_x, dd_Y, dd_W), each timed alone with HIP events on its stream."""
    gx, gY, gW = torch.randn_like(x), torch.randn_like(Y), torch.randn_like(W)
    legs = {"dd_out": ("grad_out",), "dd_x_Y_W": ("x", "Y", "W")}
    res = {}
    for name, want in legs.items():
        for _ in range(3):
            plan.conv_bwd_bwd(rp, src, x, Y, W, G, gx, gY, gW, ws, want=want)
        ts = []
        for _ in range(max(5, steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            plan.conv_bwd_bwd(rp, src, x, Y, W, G, gx, gY, gW, ws, want=want)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = statistics.median(a.elapsed_time(b) for a, b in ts)
        nbytes = ab["dbl_fwd" if name == "dd_out" else "dbl_bwd"]
        res[name] = {"ms": ms, "alg_bytes": nbytes, "alg_gbs": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del gx, gY, gW
    log(f"  double backward: dd_out {res['dd_out']['ms']:.3f} ms ({res['dd_out']['alg_gbs']:.0f} GB/s alg) | "
        f"dd_x,dd_Y,dd_W {res['dd_x_Y_W']['ms']:.3f} ms ({res['dd_x_Y_W']['alg_gbs']:.0f} GB/s alg)")
    return res


def _median_ms(torch, stream, fn, steps):
    for _ in range(3):
        fn()
    ts = []
    for _ in range(max(5, steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ts)


def time_path_outputs(torch, stream, rp, src, x, Y, W, steps):
    """The per-path (concatenated) outputs and their fully connected (uvw)
    mixing with C_out = C: median times of the convolution forward and
    backward (all launches of each call) and of the mixing forward and
    backward, HIP events on their stream.  Algorithmic bytes as for the
    summed convolution with D_mid output rows; the mixing is reported as fp64
    matrix-core TFLOP/s (2 N D_mid C C_out flops forward, twice that backward)."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan

    N, E, C = x.shape[0], Y.shape[0], x.shape[2]
    L = int(round(math.sqrt(Y.shape[1]))) - 1
    plan = Plan(L, L, L, C, path_outputs=True)
    P, Dm = plan.num_paths, plan.dim_out
    ws = plan.graph_prepare(rp, src)
    G = torch.randn((N, Dm, C), device=x.device)
    Wm = torch.randn((P, C, C), device=x.device) / math.sqrt(C)
    mid = torch.empty((N, Dm, C), device=x.device)
    res = {"d_mid": Dm}
    res["fwd_ms"] = _median_ms(torch, stream, lambda: plan.conv_fwd(rp, src, x, Y, W, ws, out=mid), steps)
    res["bwd_ms"] = _median_ms(torch, stream, lambda: plan.conv_bwd(rp, src, x, Y, W, G, ws), steps)
    fwd_b = E * (4 * P * C + 4 * plan.dim_sh + 4) + N * (4 * C * (plan.dim_in + Dm) + 4)
    bwd_b = E * (8 * P * C + 8 * plan.dim_sh + 8) + N * (4 * C * (2 * plan.dim_in + Dm) + 4)
    res["fwd_alg_gbs"] = fwd_b / (res["fwd_ms"] * 1e-3) / 1e9
    res["bwd_alg_gbs"] = bwd_b / (res["bwd_ms"] * 1e-3) / 1e9
    Gz = torch.randn((N, plan.dim_z, C), device=x.device)
    res["mix_fwd_ms"] = _median_ms(torch, stream, lambda: plan.path_mix_fwd(mid, Wm), steps)
    res["mix_bwd_ms"] = _median_ms(torch, stream, lambda: plan.path_mix_bwd(mid, Wm, Gz), steps)
    fl = 2.0 * N * Dm * C * C
    res["mix_fwd_tflops"] = fl / (res["mix_fwd_ms"] * 1e-3) / 1e12
    res["mix_bwd_tflops"] = 2 * fl / (res["mix_bwd_ms"] * 1e-3) / 1e12
    log(f"  per-path outputs (D_mid {Dm}): fwd {res['fwd_ms']:.3f} ms | bwd {res['bwd_ms']:.3f} ms | uvw mixing fwd "
        f"{res['mix_fwd_ms']:.3f} ms ({res['mix_fwd_tflops']:.1f} TFLOP/s) bwd {res['mix_bwd_ms']:.3f} ms "
        f"({res['mix_bwd_tflops']:.1f} TFLOP/s)")
    del ws, G, Wm, mid, Gz
    return res


def cp_alg_bytes(N, E, C, d_in, d_sh, d_out):
    """Bytes the CP convolution must move: forward reads x, Y, one weight per
    edge and channel, the CSR, and writes out; backward reads x, grad_out, Y,
    W, the view and writes grad_x, grad_W, grad_Y (the projected rows are the
    implementation's own traffic, not counted)."""
    fwd = E * (4 * C + 4 * d_sh + 4) + N * (4 * C * (d_in + d_out) + 4)
    bwd = E * (8 * C + 8 * d_sh + 8) + N * (4 * C * (2 * d_in + d_out) + 4)
    return fwd, bwd


def time_cp(torch, plan, stream, rp, src, x, Y, G, ranks, steps):
    """The CP-decomposed convolution (one weight per edge and channel) with
    factors from the library's data-free fit: median times of the whole
    forward and backward calls (projections included), HIP events on their
    stream."""
    import numpy as np

    N, E, C = x.shape[0], Y.shape[0], plan.channels
    W = torch.randn((E, C), device=x.device) / math.sqrt(plan.num_paths)
    fb, bb = cp_alg_bytes(N, E, C, plan.dim_in, plan.dim_sh, plan.dim_out)
    out = {}
    for R in ranks:
        rng = np.random.default_rng(R)
        A, B, Cf, err = plan.cp_fit(rng.standard_normal((plan.dim_out, R)), rng.standard_normal((plan.dim_in, R)),
                                    rng.standard_normal((plan.dim_sh, R)), sweeps=200)
        fA, fB, fC = (torch.from_numpy(v.astype(np.float32)).to(x.device) for v in (A, B, Cf))
        ws = torch.empty(plan.cp_workspace_size(R, N, E), dtype=torch.uint8, device=x.device)
        plan.graph_prepare(rp, src, ws)
        o = torch.empty((N, plan.dim_out, C), device=x.device)
        res = {"fit_rel_err": err}
        for name, fn in (("fwd", lambda: plan.cp_conv_fwd(rp, src, x, Y, W, fA, fB, fC, ws, out=o)),
                         ("bwd", lambda: plan.cp_conv_bwd(rp, src, x, Y, W, fA, fB, fC, G, ws))):
            for _ in range(3):
                fn()
            ts = []
            for _ in range(max(5, steps)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            ms = statistics.median(a.elapsed_time(b) for a, b in ts)
            nb = fb if name == "fwd" else bb
            res[name + "_ms"] = ms
            res[name + "_alg_gbs"] = nb / (ms * 1e-3) / 1e9
        res["fwd_bwd_edges_per_s"] = E / ((res["fwd_ms"] + res["bwd_ms"]) * 1e-3)
        out[str(R)] = res
        log(f"  CP rank {R} (fit error {err:.1e}): fwd {res['fwd_ms']:.3f} ms | bwd {res['bwd_ms']:.3f} ms")
        del ws, o
    return out


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, g, x, W, G, min_seconds=10.0):
    """The fp64 oracle on full steps of the headline workload (host cores),
    repeated until about `min_seconds` of CPU work has been timed, plus a
    one-thread sample in a child process."""
    import numpy as np

    import oracle

    L = w.l_max
    steps = 0
    t0 = time.perf_counter()
    while True:
        Y = oracle.sh(L, g.r)
        oracle.graph_transpose(g.row_ptr, g.src)
        Yf = Y.astype(np.float32)
        oracle.conv_fwd(L, L, L, g.row_ptr, g.src, x, Yf, W)
        oracle.conv_bwd(L, L, L, g.row_ptr, g.src, x, Yf, W, G)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    res = {"value": steps * g.n_edges / dt, "unit": "edges/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{steps} full steps (SH, transpose, fwd, bwd) of the {w.key} workload "
                     f"({g.n_edges} edges each), {dt:.1f} s",
           "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-single", w.key], env=env,
                       capture_output=True, text=True, timeout=300)
    if p.returncode == 0 and p.stdout.strip():
        res["single_thread"] = json.loads(p.stdout.strip().splitlines()[-1])
    else:
        res["single_thread"] = {"error": p.stderr[-300:]}
    return res


def cpu_single(key, seconds=4.0):
    """The oracle on one thread: whole steps over the in-edges of the first
    receivers of workload `key` (a bounded sample), edges/s."""
    import numpy as np

    import oracle
    from clebsch_gordan_tensor_cgtp_amd import synth

    w = synth.WORKLOADS[key]
    g = synth.make_graph(w)
    N, E, L, C = g.n_nodes, g.n_edges, w.l_max, w.channels
    x, W, G = synth.make_tensors_numpy(N, E, L, C)
    R = max(1, N // 50)                      # receivers in the sample
    e1 = int(g.row_ptr[R])
    rp = np.minimum(g.row_ptr, e1)
    src, r, Ws = g.src[:e1], g.r[:e1], W[:e1]
    steps = 0
    t0 = time.perf_counter()
    while True:
        Yf = oracle.sh(L, r).astype(np.float32)
        oracle.graph_transpose(rp, src)
        oracle.conv_fwd(L, L, L, rp, src, x, Yf, Ws)
        oracle.conv_bwd(L, L, L, rp, src, x, Yf, Ws, G)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    print(json.dumps({"value": steps * e1 / dt, "unit": "edges/s", "cores": oracle.num_threads(),
                      "sample": f"{steps} steps over the {e1} in-edges of the first {R} receivers of {key}, "
                                f"{dt:.1f} s"}))


def copy_ceiling(torch, dev, nbytes=2 << 30, reps=20, settle=1.0):
    """Best-of-`reps` rates of plain device copies of `nbytes`: the runtime's
    device-to-device copy and an elementwise kernel, read + write bytes, each
    after `settle` seconds of the same copy so that the clocks have settled."""
    a = torch.randn(nbytes // 4, device=dev)
    b = torch.empty_like(a)
    res = {}
    for name, fn in (("memcpy_d2d", lambda: b.copy_(a)), ("elementwise_neg", lambda: torch.neg(a, out=b))):
        t0 = time.time()
        while time.time() - t0 < settle:
            fn()
            torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name + "_gbs"] = 2 * nbytes / best / 1e6
    res["bytes_each_way"] = nbytes
    return res


# ---------------------------------------------------------------------------
# profile summaries (rocprofv3 CSV -> profiles/*.txt)
# ---------------------------------------------------------------------------
def _trace(path):
    rows = list(csv.DictReader(open(path)))
    d = {}
    for r in rows:
        d.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return d


def _pmc(path):
    rows = list(csv.DictReader(open(path)))
    d = {}
    for r in rows:
        d.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in d.items()}


def _short(name):
    return name.replace("void ", "").replace("(anonymous namespace)::", "").replace("cgtp::", "").split("(")[0]


# the step's forward and backward kernels by name: k_conv_fwd<LM, LPE, H, SUB, DBL, FSH, PS> and
# k_conv_bwd<LM, LPE, H, SUB, DBL, MID, FSH, PS> with DBL, MID and FSH false (PS, the path-split
# form, is the degree-3 step's backward)
STEP_KERNEL = {"conv_fwd": r"k_conv_fwd<\d+, \d+, \d+, (true|false), false, false, (true|false)>",
               "conv_bwd": r"k_conv_bwd<\d+, \d+, \d+, (true|false), false, false, false, (true|false)>"}


def summarize(d, workload):
    """Write profiles/{kernel_trace,pmc_conv_fwd,pmc_conv_bwd,sq}_<workload>.txt
    from the rocprofv3 output under `d` (subdirectories named as in the
    commands each summary lists)."""
    cmd = f"python3 bench.py --workloads {workload} --steps 10 --warmup 2 --settle 0.3 --no-cpu-baseline"
    cmd_pmc = cmd + " --no-extras"
    def find(sub, f):
        # the copy calibration may sit beside the workload's directory
        for base in (d, os.path.dirname(os.path.normpath(d))):
            if os.path.exists(os.path.join(base, sub, f)):
                return os.path.join(base, sub, f)
        return os.path.join(d, sub, f)
    out = os.path.join(ROOT, "profiles")
    sha = kernel_source_sha()
    # kernel trace
    tr = _trace(find("trace", "run_kernel_trace.csv"))
    lines = [f"# rocprofv3 kernel trace of bench.py on the {workload} workload",
             f"# command (repo root): rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- {cmd}",
             "# per-dispatch durations in microseconds (end - start) over every dispatch of the run",
             f"{'kernel':52s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_%':>8s}"]
    tot = sum(sum(v) for v in tr.values())
    for k, v in sorted(tr.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{_short(k)[:52]:52s} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):9.2f} "
                     f"{min(v):9.2f} {max(v):9.2f} {100 * sum(v) / tot:8.2f}")
    lines.append(f"kernel_source_sha = {sha}")
    open(os.path.join(out, f"kernel_trace_{workload}.txt"), "w").write("\n".join(lines) + "\n")
    # HBM bytes
    fetch, write = _pmc(find("fetch", "run_counter_collection.csv")), _pmc(find("write", "run_counter_collection.csv"))
    cf, cw = _pmc(find("cal_fetch", "run_counter_collection.csv")), _pmc(find("cal_write", "run_counter_collection.csv"))
    neg = [k for k in cf if "neg_kernel" in k][0]
    gib_kib = float(1 << 20)   # 1 GiB in KiB, read and written by the calibration copy
    ff, wf = gib_kib / cf[neg]["FETCH_SIZE"], gib_kib / cw[neg]["WRITE_SIZE"]
    from clebsch_gordan_tensor_cgtp_amd import synth
    w = synth.WORKLOADS[workload]
    g = synth.make_graph(w)
    D = (w.l_max + 1) ** 2
    alg_all = algorithmic_bytes(g.n_nodes, g.n_edges, w.num_paths, w.channels, D, D, D)
    for kern in ("conv_fwd", "conv_bwd"):
        # the step's kernel (the double backward, the per-path outputs and the fused-SH
        # forms instantiate the same template with DBL, MID or FSH = true)
        name = [k for k in fetch if re.search(STEP_KERNEL[kern], k)][0]
        fk, wk = fetch[name]["FETCH_SIZE"], write[name]["WRITE_SIZE"]
        rd, wr = fk * 1024 * ff, wk * 1024 * wf
        alg = alg_all[kern.split("_")[1]]
        lines = [f"# HBM traffic of {_short(name)} on the {workload} workload ({w.name})",
                 "# commands (repo root; one counter per pass):",
                 f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- {cmd_pmc}",
                 f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- {cmd_pmc}",
                 "# calibration on a plain copy of known size (torch neg() over 1 GiB fp32: 1 GiB read + 1 GiB written):",
                 "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/cal_fetch -o run -- python3 bench.py --copy-calibration",
                 "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/cal_write -o run -- python3 bench.py --copy-calibration",
                 f"# copy: FETCH_SIZE {cf[neg]['FETCH_SIZE']:.1f} KiB, WRITE_SIZE {cw[neg]['WRITE_SIZE']:.1f} KiB "
                 f"per launch for 1048576 KiB each way (medians over launches)",
                 f"fetch_factor = {ff:.4f}", f"write_factor = {wf:.4f}",
                 f"fetch_kib_raw = {fk:.1f}", f"write_kib_raw = {wk:.1f}",
                 f"read_bytes_per_launch = {rd:.0f}", f"write_bytes_per_launch = {wr:.0f}",
                 f"hbm_bytes_per_launch = {rd + wr:.0f}",
                 f"algorithmic_bytes_per_launch = {alg}", f"traffic_over_algorithmic = {(rd + wr) / alg:.3f}"]
        lines += [f"kernel_source_sha = {sha}",
                  "# kernel_source_sha: first 16 hex digits of sha256 over cgtp_kernels.h + cgtp_math.h + cgtp_sh.h;",
                  "# bench.py reports traffic only while the sources still hash to this value"]
        open(os.path.join(out, f"pmc_{kern}_{workload}.txt"), "w").write("\n".join(lines) + "\n")
    # instruction issue (SQ) counters
    sq = _pmc(find("sq1", "run_counter_collection.csv"))
    sq2 = _pmc(find("sq2", "run_counter_collection.csv"))
    lines = [f"# SQ / GRBM counters of the convolution kernels on the {workload} workload (medians over launches)",
             "# commands (repo root):",
             f"#   rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
             f"SQ_ACTIVE_INST_VALU SQ_INSTS_VALU GRBM_GUI_ACTIVE GRBM_COUNT --output-format csv -d <dir>/sq1 -o run -- {cmd_pmc}",
             f"#   rocprofv3 --pmc SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR "
             f"SQ_INSTS_SALU SQ_INST_CYCLES_VMEM_RD SQ_WAIT_INST_LDS --output-format csv -d <dir>/sq2 -o run -- {cmd_pmc}",
             "# derived (per launch): gpu_cycles = GRBM_GUI_ACTIVE / 8 (one count per XCD); VALU busy =",
             "# 4 * SQ_ACTIVE_INST_VALU / (gpu_cycles * 1024 SIMDs) (SQ cycle counters count 4-cycle units);",
             "# mean resident waves per SIMD = 4 * SQ_WAVE_CYCLES / (gpu_cycles * 1024)"]
    for name, c in sq.items():
        if not any(re.search(p, name) for p in STEP_KERNEL.values()):
            continue
        c = dict(c)
        c.update(sq2.get(name, {}))
        cyc = c["GRBM_GUI_ACTIVE"] / 8
        lines.append(f"[{_short(name)}]")
        for k in sorted(c):
            lines.append(f"{k} = {c[k]:.0f}")
        lines.append(f"gpu_cycles = {cyc:.0f}")
        lines.append(f"valu_busy = {4 * c['SQ_ACTIVE_INST_VALU'] / (cyc * 1024):.3f}")
        lines.append(f"resident_waves_per_simd = {4 * c['SQ_WAVE_CYCLES'] / (cyc * 1024):.2f}")
        lines.append(f"valu_insts_per_wave = {c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.1f}")
    lines.append(f"kernel_source_sha = {sha}")
    open(os.path.join(out, f"sq_{workload}.txt"), "w").write("\n".join(lines) + "\n")
    log(f"wrote profiles for {workload}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="extra untimed warm-up, in seconds of sustained load, after the --warmup steps")
    ap.add_argument("--workloads", default=",".join([HEADLINE] + OTHERS),
                    help="comma list; the first is the headline (value)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (skip the double-backward and CP legs)")
    ap.add_argument("--locality", action="store_true",
                    help="schedule blocks by graph-derived clusters per XCD instead of longest first")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy kernel (PMC byte calibration)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="measure only the device-to-device copy rate (the practical HBM ceiling)")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 output in DIR")
    ap.add_argument("--cpu-single", metavar="KEY", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU sharding is "
              "not built", file=sys.stderr)
        sys.exit(2)
    if args.cpu_single:
        cpu_single(args.cpu_single)
        return
    keys = args.workloads.split(",")
    if args.summarize:
        summarize(args.summarize, keys[0])
        return

    import torch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = (1 << 30) // 4
        a = torch.randn(n, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 launches of neg(), {4 * n} bytes read and {4 * n} written per launch")
        return
    if args.copy_ceiling:
        print(json.dumps(copy_ceiling(torch, dev)), flush=True)
        return

    extras = not args.no_extras
    head, host = run_workload(torch, dev, keys[0], args.steps, args.warmup, args.settle, args.locality, extras)
    others = {}
    for k in keys[1:]:
        others[k], _ = run_workload(torch, dev, k, max(5, args.steps // 2), 2, args.settle, args.locality, extras)

    kern, kms, kbytes = "conv_bwd", head["bwd_ms"], head["alg_bytes"]["bwd"]
    achieved = kbytes / (kms * 1e-3) / 1e9
    config = {"workload": head["workload"], "storage": "f32",
              "step": "sh + graph_prepare + conv_fwd + conv_bwd(dx, dW, dY)",
              "schedule": "locality" if args.locality else "longest-first"}
    config.update({k: v for k, v in head.items() if k not in ("workload",)})
    res = {
        "metric": "CGTP conv fwd+bwd edges/sec and achieved HBM GB/s (% peak), L=2 C=128 fp32",
        "value": head["edges_per_s"],
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "kernel": kern, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic(kern, keys[0]),
            "alg_bytes_per_launch": kbytes, "median_launch_ms": kms,
            "timing": "median over the timed steps of HIP events around the launch on its stream",
        },
        "workloads": others,
    }
    if not args.no_cpu_baseline and host is not None:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(*host)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
