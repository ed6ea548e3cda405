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

    def __init__(self, l_in: int, l_sh: int, l_out: int, channels: int, validate: bool = False):
        lib = L.lib()
        h = ctypes.c_void_p()
        flags = L.CGTP_FLAG_VALIDATE if validate else 0
        L.check("cgtp_plan_create", lib.cgtp_plan_create(ctypes.byref(h), l_in, l_sh, l_out, channels, flags))
        self._h = h
        self.l_in, self.l_sh, self.l_out, self.channels = l_in, l_sh, l_out, channels
        P, di, ds, do = (ctypes.c_int() for _ in range(4))
        L.check("cgtp_plan_info", lib.cgtp_plan_info(h, ctypes.byref(P), None, ctypes.byref(di),
                                                      ctypes.byref(ds), ctypes.byref(do)))
        self.num_paths = P.value
        self.dim_in, self.dim_sh, self.dim_out = di.value, ds.value, do.value
        arr = (ctypes.c_int * (3 * self.num_paths))()
        L.check("cgtp_plan_info", lib.cgtp_plan_info(h, None, arr, None, None, None))
        self.paths = [tuple(arr[3 * q:3 * q + 3]) for q in range(self.num_paths)]

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

    def conv_fwd(self, row_ptr, src, x, Y, W, ws, out=None) -> torch.Tensor:
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), dev)
        _need(W, "W", torch.float32, (E, self.num_paths, C), dev)
        _need(ws, "ws", torch.uint8, device=dev)
        if out is None:
            out = torch.empty((N, self.dim_out, C), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (N, self.dim_out, C), dev)
        L.check("cgtp_conv_fwd", L.lib().cgtp_conv_fwd(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(out), _ptr(ws),
            ws.numel(), _stream(dev)))
        return out

    def conv_bwd(self, row_ptr, src, x, Y, W, grad_out, ws, want=("dx", "dW", "dY"),
                 grad_x=None, grad_W=None, grad_Y=None):
        """(grad_x, grad_W, grad_Y); a gradient not in ``want`` comes back as None."""
        N, E, C, dev = row_ptr.shape[0] - 1, src.shape[0], self.channels, row_ptr.device
        _need(row_ptr, "row_ptr", torch.int32)
        _need(src, "src", torch.int32, (E,), dev)
        _need(x, "x", torch.float32, (N, self.dim_in, C), dev)
        _need(Y, "Y", torch.float32, (E, self.dim_sh), dev)
        _need(W, "W", torch.float32, (E, self.num_paths, C), dev)
        _need(grad_out, "grad_out", torch.float32, (N, self.dim_out, C), dev)
        _need(ws, "ws", torch.uint8, device=dev)
        if "dx" in want and grad_x is None:
            grad_x = torch.empty((N, self.dim_in, C), dtype=torch.float32, device=dev)
        if "dW" in want and grad_W is None:
            grad_W = torch.empty((E, self.num_paths, C), dtype=torch.float32, device=dev)
        if "dY" in want and grad_Y is None:
            grad_Y = torch.empty((E, self.dim_sh), dtype=torch.float32, device=dev)
        if "dx" not in want:
            grad_x = None
        if "dW" not in want:
            grad_W = None
        if "dY" not in want:
            grad_Y = None
        for t, n, s in ((grad_x, "grad_x", (N, self.dim_in, C)), (grad_W, "grad_W", (E, self.num_paths, C)),
                        (grad_Y, "grad_Y", (E, self.dim_sh))):
            if t is not None:
                _need(t, n, torch.float32, s, dev)
        L.check("cgtp_conv_bwd", L.lib().cgtp_conv_bwd(
            self._h, N, E, _ptr(row_ptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W), _ptr(grad_out),
            _ptr(grad_x), _ptr(grad_W), _ptr(grad_Y), _ptr(ws), ws.numel(), _stream(dev)))
        return grad_x, grad_W, grad_Y
