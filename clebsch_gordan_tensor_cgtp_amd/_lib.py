"""ctypes binding of libcgtp.so (the C ABI declared in include/cgtp.h).

Argument marshalling only: every step of the convolution runs in the HIP
kernels of libcgtp.so.  torch is imported first so that the library binds to
the HIP runtime torch already loaded (both carry the soname libamdhip64.so.7),
which lets it use torch's device memory and streams.  There is no fallback:
a missing library raises.
"""
import ctypes
import os

import torch  # noqa: F401  (must precede loading libcgtp.so; see module docstring)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcgtp.so")

CGTP_OK = 0
CGTP_ERR_INVALID_ARG = -1
CGTP_ERR_UNSUPPORTED = -2
CGTP_ERR_WORKSPACE = -3
CGTP_ERR_HIP = -4
CGTP_ERR_ALLOC = -5
CGTP_ERR_GRAPH = -6
CGTP_ERR_NUMERIC = -7
CGTP_FLAG_VALIDATE = 1
CGTP_FLAG_LOCALITY = 2
CGTP_FLAG_SHARED_WEIGHTS = 4
CGTP_FLAG_PATH_OUTPUTS = 8

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes); mirrors include/cgtp.h
SIGNATURES = {
    "cgtp_plan_create": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_uint]),
    "cgtp_plan_destroy": (ctypes.c_int, [_vp]),
    "cgtp_plan_info": (ctypes.c_int, [_vp, _ip, _ip, _ip, _ip, _ip]),
    "cgtp_plan_export_cg": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]),
    "cgtp_workspace_size": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "cgtp_sh_fwd": (ctypes.c_int, [_vp, _c_i64, _vp, _vp, _vp]),
    "cgtp_sh_bwd": (ctypes.c_int, [_vp, _c_i64, _vp, _vp, _vp, _vp]),
    "cgtp_node_grad": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "cgtp_graph_prepare": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "cgtp_conv_fwd": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                     _vp]),
    "cgtp_conv_bwd": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, ctypes.c_size_t, _vp]),
    "cgtp_conv_fwd_sh": (ctypes.c_int, [_vp, _c_i64, _c_i64] + [_vp] * 7 + [ctypes.c_size_t, _vp]),
    "cgtp_conv_bwd_sh": (ctypes.c_int, [_vp, _c_i64, _c_i64] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "cgtp_conv_bwd_bwd": (ctypes.c_int, [_vp, _c_i64, _c_i64] + [_vp] * 14 + [ctypes.c_size_t, _vp]),
    "cgtp_path_mix_workspace_size": (ctypes.c_int, [_vp, _c_i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "cgtp_path_mix_fwd": (ctypes.c_int, [_vp, _c_i64, ctypes.c_int, _vp, _vp, _vp, _vp]),
    "cgtp_path_mix_bwd": (ctypes.c_int, [_vp, _c_i64, ctypes.c_int] + [_vp] * 6 + [ctypes.c_size_t, _vp]),
    "cgtp_cp_workspace_size": (ctypes.c_int, [_vp, ctypes.c_int, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "cgtp_cp_fit": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_double] + [_vp] * 4),
    "cgtp_cp_conv_fwd": (ctypes.c_int, [_vp, ctypes.c_int, _c_i64, _c_i64] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "cgtp_cp_conv_bwd": (ctypes.c_int, [_vp, ctypes.c_int, _c_i64, _c_i64] + [_vp] * 13 + [ctypes.c_size_t, _vp]),
    "cgtp_conv_bwd_noalloc": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp]),
    "cgtp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class CgtpError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib():
    """The loaded libcgtp.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcgtp.so not found at {LIB_PATH}; build it with "
                           "`python -m clebsch_gordan_tensor_cgtp_amd.build`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(handle, name)
        f.restype = res
        f.argtypes = args
    _lib = handle
    return handle


def status_string(status: int) -> str:
    return lib().cgtp_status_string(int(status)).decode()


def check(fn: str, status: int):
    if status != CGTP_OK:
        raise CgtpError(fn, status)
