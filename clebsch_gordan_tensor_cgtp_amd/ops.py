"""Python face of libcgtp.so: a Plan object whose methods take torch tensors.

Each method checks dtypes, devices and shapes, allocates outputs with torch
(device memory only) and calls the C ABI on the current HIP stream.  No
arithmetic of the convolution happens here.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class Plan:
    """Compiled CGTP convolution for degrees (l_in, l_sh, l_out) and C channels."""

    def __init__(self, l_in: int, l_sh: int, l_out: int, channels: int, validate: bool = False,
                 locality: bool = False, shared_weights: bool = False, path_outputs: bool = False):
        """path_outputs: every path keeps its own 2*l3+1 output rows (out and
        grad_out are [N][dim_out][C] with dim_out = sum over paths of 2*l3+1)."""
        lib = L.lib()
        h = ctypes.c_void_p()
        flags = (L.CGTP_FLAG_VALIDATE if validate else 0) | (L.CGTP_FLAG_LOCALITY if locality else 0) | \
            (L.CGTP_FLAG_SHARED_WEIGHTS if shared_weights else 0) | (L.CGTP_FLAG_PATH_OUTPUTS if path_outputs else 0)
        self.path_outputs = path_outputs
        self.shared_weights = shared_weights
        L.check("cgtp_plan_create", lib.cgtp_plan_create(ctypes.byref(h), l_in, l_sh, l_out, channels, flags))
        self._h = h
        self.l_in, self.l_sh, self.l_out, self.channels = l_in, l_sh, l_out, channels
        P, di, ds, do = (ctypes.c_int() for _ in range(4))
        L.check("cgtp_plan_info", lib.cgtp_plan_info(h, ctypes.byref(P), None, ctypes.byref(di),
                                                      ctypes.byref(ds), ctypes.byref(do)))
        self.num_paths = P.value
        self.dim_in, self.dim_sh, self.dim_out = di.value, ds.value, do.value
        self.dim_z = (l_out + 1) ** 2   # the coupled output's width (the CP product's d3)
        arr = (ctypes.c_int * (3 * self.num_paths))()
        L.check("cgtp_plan_info", lib.cgtp_plan_info(h, None, arr, None, None, None))
        self.paths = [tuple(arr[3 * q:3 * q + 3]) for q in range(self.num_paths)]
        self.weight_rows = 1 if shared_weights else self.num_paths   # W is [E][weight_rows][C]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and L._lib is not None:
            L._lib.cgtp_plan_destroy(h)
            self._h = None

    # -- host-side queries ---------------------------------------------------
    def export_cg(self, path: int) -> np.ndarray:
        l1, l2, l3 = self.paths[path]
        out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1), dtype=np.float64)
        L.check("cgtp_plan_export_cg",
                L.lib().cgtp_plan_export_cg(self._h, path, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
        return out

    def workspace_size(self, n_nodes: int, n_edges: int) -> int:
        b = ctypes.c_size_t()
        L.check("cgtp_workspace_size", L.lib().cgtp_workspace_size(self._h, n_nodes, n_edges, ctypes.byref(b)))
        return b.value

    # -- device calls --------------------------------------------------------
    def sh(self, r: torch.Tensor, Y: torch.Tensor | None = None) -> torch.Tensor:
        E = r.shape[0]
        _need(r, "r", torch.float32, (E, 3))
        if Y is None:
            Y = torch.empty((E, self.dim_sh), dtype=torch.float32, device=r.device)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), r.device)
        L.check("cgtp_sh_fwd", L.lib().cgtp_sh_fwd(self._h, E, _ptr(r), _ptr(Y), _stream(r.device)))
        return Y

    def sh_bwd(self, r: torch.Tensor, grad_Y: torch.Tensor, grad_r: torch.Tensor | None = None) -> torch.Tensor:
        """grad_r[E][3] = grad_Y[e] . dY/dr at r[e]."""
        E = r.shape[0]
        _need(r, "r", torch.float32, (E, 3))
        _need(grad_Y, "grad_Y", torch.float32, (E, self.dim_sh), r.device)
        if grad_r is None:
            grad_r = torch.empty((E, 3), dtype=torch.float32, device=r.device)
        _need(grad_r, "grad_r", torch.float32, (E, 3), r.device)
        L.check("cgtp_sh_bwd", L.lib().cgtp_sh_bwd(self._h, E, _ptr(r), _ptr(grad_Y), _ptr(grad_r),
                                                   _stream(r.device)))
        return grad_r

    def node_grad(self, row_ptr, src, grad_r, ws=None, grad_pos=None) -> torch.Tensor:
        """grad_pos[N][3] from per-edge gradients of r = pos[src] - pos[dst]."""
        N, E, dev = row_ptr.shape[0] - 1, src.shape[0], row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(grad_r, "grad_r", torch.float32, (E, 3), dev)
        ws = self._workspace(ws, row_ptr, src)
        if grad_pos is None:
            grad_pos = torch.empty((N, 3), dtype=torch.float32, device=dev)
        _need(grad_pos, "grad_pos", torch.float32, (N, 3), dev)
        L.check("cgtp_node_grad", L.lib().cgtp_node_grad(self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(grad_r),
                                                         _ptr(grad_pos), _ptr(ws), ws.numel(), _stream(dev)))
        return grad_pos

    def graph_prepare(self, row_ptr: torch.Tensor, src: torch.Tensor,
                      ws: torch.Tensor | None = None) -> torch.Tensor:
        N, E = row_ptr.shape[0] - 1, src.shape[0]
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, device=row_ptr.device)
        nbytes = self.workspace_size(N, E)
        if ws is None:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=row_ptr.device)
        _need(ws, "ws", torch.uint8, device=row_ptr.device)
        L.check("cgtp_graph_prepare", L.lib().cgtp_graph_prepare(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(ws), ws.numel(), _stream(row_ptr.device)))
        return ws

    def _workspace(self, ws, row_ptr, src):
        # A workspace allocated here is prepared here: the library knows a
        # prepared workspace by its address, and a fresh allocation can land
        # where an earlier, since freed, workspace of the same graph was.
        if ws is None:
            return self.graph_prepare(row_ptr, src)
        _need(ws, "ws", torch.uint8, device=row_ptr.device)
        return ws

    def conv_fwd(self, row_ptr, src, x, Y, W, ws=None, out=None) -> torch.Tensor:
        """out[N][D_out][C].  ``ws``: the graph's workspace (from graph_prepare,
        or any buffer of workspace_size bytes, which the call then prepares
        unless it already holds this graph's view; a buffer whose memory
        served anything else since its preparation must be prepared again).
        Without ``ws`` a workspace is allocated and prepared for this call."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), dev)
        _need(W, "W", torch.float32, (E, self.weight_rows, C), dev)
        ws = self._workspace(ws, row_ptr, src)
        if out is None:
            out = torch.empty((N, self.dim_out, C), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (N, self.dim_out, C), dev)
        L.check("cgtp_conv_fwd", L.lib().cgtp_conv_fwd(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(out), _ptr(ws),
            ws.numel(), _stream(dev)))
        return out

    def conv_bwd(self, row_ptr, src, x, Y, W, grad_out, ws=None, want=("dx", "dW", "dY"),
                 grad_x=None, grad_W=None, grad_Y=None):
        """(grad_x, grad_W, grad_Y); a gradient not in ``want`` comes back as None."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), dev)
        _need(W, "W", torch.float32, (E, self.weight_rows, C), dev)
        _need(grad_out, "grad_out", torch.float32, (N, self.dim_out, C), dev)
        ws = self._workspace(ws, row_ptr, src)
        if "dx" in want and grad_x is None:
            grad_x = torch.empty((N, self.dim_in, C), dtype=torch.float32, device=dev)
        if "dW" in want and grad_W is None:
            grad_W = torch.empty((E, self.weight_rows, C), dtype=torch.float32, device=dev)
        if "dY" in want and grad_Y is None:
            grad_Y = torch.empty((E, self.dim_sh), dtype=torch.float32, device=dev)
        if "dx" not in want:
            grad_x = None
        if "dW" not in want:
            grad_W = None
        if "dY" not in want:
            grad_Y = None
        for t, n, s in ((grad_x, "grad_x", (N, self.dim_in, C)), (grad_W, "grad_W", (E, self.weight_rows, C)),
                        (grad_Y, "grad_Y", (E, self.dim_sh))):
            if t is not None:
                _need(t, n, torch.float32, s, dev)
        L.check("cgtp_conv_bwd", L.lib().cgtp_conv_bwd(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(grad_out),
            _ptr(grad_x), _ptr(grad_W), _ptr(grad_Y), _ptr(ws), ws.numel(), _stream(dev)))
        return grad_x, grad_W, grad_Y

    def conv_fwd_sh(self, row_ptr, src, x, r, W, ws=None, out=None) -> torch.Tensor:
        """conv_fwd with the spherical harmonics evaluated inside the kernel
        from the edge vectors r [E][3] (fp64, not rounded to fp32)."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(r, "r", torch.float32, (E, 3), dev)
        _need(W, "W", torch.float32, (E, self.weight_rows, C), dev)
        ws = self._workspace(ws, row_ptr, src)
        if out is None:
            out = torch.empty((N, self.dim_out, C), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (N, self.dim_out, C), dev)
        L.check("cgtp_conv_fwd_sh", L.lib().cgtp_conv_fwd_sh(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(r), _ptr(W), _ptr(out), _ptr(ws),
            ws.numel(), _stream(dev)))
        return out

    def conv_bwd_sh(self, row_ptr, src, x, r, W, grad_out, ws=None, want=("dx", "dW", "dr")):
        """(grad_x, grad_W, grad_r) of <grad_out, conv_fwd_sh(x, r, W)>; grad_r
        [E][3] is the SH backward of the grad_Y conv_bwd would return."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(r, "r", torch.float32, (E, 3), dev)
        _need(W, "W", torch.float32, (E, self.weight_rows, C), dev)
        _need(grad_out, "grad_out", torch.float32, (N, self.dim_out, C), dev)
        ws = self._workspace(ws, row_ptr, src)
        f = lambda k, s: torch.empty(s, dtype=torch.float32, device=dev) if k in want else None
        grad_x, grad_W, grad_r = f("dx", (N, self.dim_in, C)), f("dW", (E, self.weight_rows, C)), f("dr", (E, 3))
        L.check("cgtp_conv_bwd_sh", L.lib().cgtp_conv_bwd_sh(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(r), _ptr(W), _ptr(grad_out),
            _ptr(grad_x), _ptr(grad_W), _ptr(grad_r), _ptr(ws), ws.numel(), _stream(dev)))
        return grad_x, grad_W, grad_r

    def conv_bwd_bwd(self, row_ptr, src, x, Y, W, grad_out, gg_x=None, gg_Y=None, gg_W=None, ws=None,
                     want=("x", "Y", "W", "grad_out")):
        """Double backward: the gradients (dd_x, dd_Y, dd_W, dd_out) of
        S = <gg_x, grad_x> + <gg_W, grad_W> + <gg_Y, grad_Y>, where
        (grad_x, grad_W, grad_Y) = conv_bwd(x, Y, W, grad_out), with respect to
        x, Y, W and grad_out.  A cotangent left as None is zero; a result not
        in ``want`` comes back as None."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        sx, sy, sw, so = (N, self.dim_in, C), (E, self.dim_sh), (E, self.weight_rows, C), (N, self.dim_out, C)
        _need(x, "x", torch.float32, sx, dev)
        _need(Y, "Y", torch.float32, sy, dev)
        _need(W, "W", torch.float32, sw, dev)
        _need(grad_out, "grad_out", torch.float32, so, dev)
        for t, n, s in ((gg_x, "gg_x", sx), (gg_Y, "gg_Y", sy), (gg_W, "gg_W", sw)):
            if t is not None:
                _need(t, n, torch.float32, s, dev)
        ws = self._workspace(ws, row_ptr, src)
        new = lambda shape, key: torch.empty(shape, dtype=torch.float32, device=dev) if key in want else None
        dd_x, dd_Y, dd_W, dd_out = new(sx, "x"), new(sy, "Y"), new(sw, "W"), new(so, "grad_out")
        L.check("cgtp_conv_bwd_bwd", L.lib().cgtp_conv_bwd_bwd(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(grad_out), _ptr(gg_x),
            _ptr(gg_Y), _ptr(gg_W), _ptr(dd_x), _ptr(dd_Y), _ptr(dd_W), _ptr(dd_out), _ptr(ws), ws.numel(),
            _stream(dev)))
        return dd_x, dd_Y, dd_W, dd_out

    # -- fully connected ("uvw") mixing of the per-path outputs ----------------
    @property
    def mid_rows(self) -> int:
        """Rows of the per-path outputs: sum over the paths of 2*l3+1."""
        return sum(2 * l3 + 1 for (_, _, l3) in self.paths)

    def path_mix_fwd(self, mid, Wmix, out=None) -> torch.Tensor:
        """out[N][(l_out+1)^2][C_out] = per path, mid's block times Wmix[p]
        [C][C_out], summed over the paths of each l3."""
        N, C, dev = mid.shape[0], self.channels, mid.device
        Co = Wmix.shape[2]
        _need(mid, "mid", torch.float32, (N, self.mid_rows, C))
        _need(Wmix, "Wmix", torch.float32, (self.num_paths, C, Co), dev)
        if out is None:
            out = torch.empty((N, self.dim_z, Co), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (N, self.dim_z, Co), dev)
        L.check("cgtp_path_mix_fwd", L.lib().cgtp_path_mix_fwd(self._h, N, Co, _ptr(mid), _ptr(Wmix), _ptr(out),
                                                               _stream(dev)))
        return out

    def path_mix_bwd(self, mid, Wmix, grad_out, want=("mid", "Wmix")):
        """(grad_mid, grad_Wmix) of <grad_out, path_mix_fwd(mid, Wmix)>."""
        N, C, dev = mid.shape[0], self.channels, mid.device
        Co = Wmix.shape[2]
        _need(mid, "mid", torch.float32, (N, self.mid_rows, C))
        _need(Wmix, "Wmix", torch.float32, (self.num_paths, C, Co), dev)
        _need(grad_out, "grad_out", torch.float32, (N, self.dim_z, Co), dev)
        gm = torch.empty_like(mid) if "mid" in want else None
        gw = torch.empty_like(Wmix) if "Wmix" in want else None
        b = ctypes.c_size_t()
        L.check("cgtp_path_mix_workspace_size", L.lib().cgtp_path_mix_workspace_size(self._h, N, Co, ctypes.byref(b)))
        ws = torch.empty(max(1, b.value), dtype=torch.uint8, device=dev)
        L.check("cgtp_path_mix_bwd", L.lib().cgtp_path_mix_bwd(self._h, N, Co, _ptr(mid), _ptr(Wmix), _ptr(grad_out),
                                                               _ptr(gm), _ptr(gw), _ptr(ws), ws.numel(), _stream(dev)))
        return gm, gw

    # -- CP-decomposed tensor product -------------------------------------------
    def cp_workspace_size(self, rank: int, n_nodes: int, n_edges: int) -> int:
        b = ctypes.c_size_t()
        L.check("cgtp_cp_workspace_size", L.lib().cgtp_cp_workspace_size(self._h, rank, n_nodes, n_edges,
                                                                          ctypes.byref(b)))
        return b.value

    def cp_fit(self, A0, B0, C0, sweeps: int, ridge: float = 1e-12):
        """Data-free ALS fit of the rank-R factors of the plan's coupling
        tensor from the start (A0 [d3][R], B0 [d1][R], C0 [d2][R]); host
        computation.  Returns (A, B, C, relative Frobenius error)."""
        R = A0.shape[1]
        A, B, C = (np.ascontiguousarray(v, dtype=np.float64).copy() for v in (A0, B0, C0))
        if A.shape != (self.dim_z, R) or B.shape != (self.dim_in, R) or C.shape != (self.dim_sh, R):
            raise ValueError("factor shapes must be [d_out][R], [d_in][R], [d_sh][R]")
        err = ctypes.c_double()
        dp = lambda a: ctypes.c_void_p(a.ctypes.data)
        L.check("cgtp_cp_fit", L.lib().cgtp_cp_fit(self._h, R, sweeps, ridge, dp(A), dp(B), dp(C), ctypes.byref(err)))
        return A, B, C, err.value

    def _cp_common(self, row_ptr, src, x, Y, W, A, B, C, ws):
        N, E, Ch, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        R = A.shape[1]
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, Ch), dev)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), dev)
        _need(W, "W", torch.float32, (E, Ch), dev)
        _need(A, "A", torch.float32, (self.dim_z, R), dev)
        _need(B, "B", torch.float32, (self.dim_in, R), dev)
        _need(C, "C", torch.float32, (self.dim_sh, R), dev)
        if ws is None:
            ws = torch.empty(self.cp_workspace_size(R, N, E), dtype=torch.uint8, device=dev)
            self.graph_prepare(row_ptr, src, ws)   # see _workspace
        _need(ws, "ws", torch.uint8, device=dev)
        return N, E, Ch, dev, R, ws

    def cp_conv_fwd(self, row_ptr, src, x, Y, W, A, B, C, ws=None, out=None) -> torch.Tensor:
        """CP convolution out[N][D_out][C]: W [E][C]; factors A [D_out][R],
        B [D_in][R], C [D_sh][R] (fp32, on the device)."""
        N, E, Ch, dev, R, ws = self._cp_common(row_ptr, src, x, Y, W, A, B, C, ws)
        if out is None:
            out = torch.empty((N, self.dim_z, Ch), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (N, self.dim_z, Ch), dev)
        L.check("cgtp_cp_conv_fwd", L.lib().cgtp_cp_conv_fwd(
            self._h, R, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(A), _ptr(B), _ptr(C),
            _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
        return out

    def cp_conv_bwd(self, row_ptr, src, x, Y, W, A, B, C, grad_out, ws=None, want=("dx", "dW", "dY")):
        """(grad_x [N][D_in][C], grad_W [E][C], grad_Y [E][D_sh]) of the CP
        convolution; a gradient not in ``want`` comes back as None."""
        N, E, Ch, dev, R, ws = self._cp_common(row_ptr, src, x, Y, W, A, B, C, ws)
        _need(grad_out, "grad_out", torch.float32, (N, self.dim_z, Ch), dev)
        new = lambda shape, key: torch.empty(shape, dtype=torch.float32, device=dev) if key in want else None
        dx, dW, dY = new((N, self.dim_in, Ch), "dx"), new((E, Ch), "dW"), new((E, self.dim_sh), "dY")
        L.check("cgtp_cp_conv_bwd", L.lib().cgtp_cp_conv_bwd(
            self._h, R, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(A), _ptr(B), _ptr(C),
            _ptr(grad_out), _ptr(dx), _ptr(dW), _ptr(dY), _ptr(ws), ws.numel(), _stream(dev)))
        return dx, dW, dY
