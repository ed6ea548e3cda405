"""Host-side checks of libcgtp.so: it loads, exports every symbol the header
declares, builds plans, reports the path list, carries CG tables equal to the
oracle's entry by entry, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from clebsch_gordan_tensor_cgtp_amd import _lib
    _lib.lib()
    return _lib


def header_functions():
    text = open(os.path.join(ROOT, "include", "cgtp.h")).read()
    return sorted(set(re.findall(r"^(?:cgtp_status_t|const char\*)\s+(cgtp_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 10
    for n in names:
        assert hasattr(L.lib(), n), n
        assert n in L.SIGNATURES, n


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_string(s) not in ("", "unknown status")
    assert L.status_string(7) == "unknown status"


def _create(L, *args):
    h = ctypes.c_void_p()
    st = L.lib().cgtp_plan_create(ctypes.byref(h), *args)
    return st, h


def test_plan_create_arguments(L):
    assert L.lib().cgtp_plan_create(None, 2, 2, 2, 128, 0) == L.CGTP_ERR_INVALID_ARG
    assert _create(L, -1, 2, 2, 128, 0)[0] == L.CGTP_ERR_INVALID_ARG
    assert _create(L, 2, 2, 2, 0, 0)[0] == L.CGTP_ERR_INVALID_ARG
    assert _create(L, 2, 2, 2, 128, 8)[0] == L.CGTP_ERR_INVALID_ARG
    assert _create(L, 4, 4, 4, 16, 0)[0] == L.CGTP_ERR_UNSUPPORTED
    assert _create(L, 2, 2, 2, 96, 0)[0] == L.CGTP_ERR_UNSUPPORTED
    assert _create(L, 3, 3, 3, 128, 0)[0] == L.CGTP_ERR_UNSUPPORTED
    for Lx, C in ((1, 8), (1, 128), (2, 8), (2, 64), (2, 128), (3, 8), (3, 64)):
        st, h = _create(L, Lx, Lx, Lx, C, 0)
        assert st == L.CGTP_OK
        assert L.lib().cgtp_plan_destroy(h) == L.CGTP_OK
    assert L.lib().cgtp_plan_destroy(None) == L.CGTP_OK


@pytest.mark.parametrize("Lx", [1, 2, 3])
def test_plan_paths_and_tables_match_oracle(L, oracle, Lx):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(Lx, Lx, Lx, 8)
    assert plan.paths == [tuple(int(v) for v in p) for p in oracle.paths(Lx, Lx, Lx)]
    assert (plan.dim_in, plan.dim_sh, plan.dim_out) == ((Lx + 1) ** 2,) * 3
    for q, (l1, l2, l3) in enumerate(plan.paths):
        got = plan.export_cg(q)
        want = oracle.real_cg(l1, l2, l3)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
        # identical nonzero pattern
        np.testing.assert_array_equal(got != 0, want != 0)


def test_export_bad_path(L):
    st, h = _create(L, 2, 2, 2, 8, 0)
    buf = (ctypes.c_double * 125)()
    assert L.lib().cgtp_plan_export_cg(h, 15, buf) == L.CGTP_ERR_INVALID_ARG
    assert L.lib().cgtp_plan_export_cg(h, -1, buf) == L.CGTP_ERR_INVALID_ARG
    assert L.lib().cgtp_plan_export_cg(None, 0, buf) == L.CGTP_ERR_INVALID_ARG
    L.lib().cgtp_plan_destroy(h)


def test_workspace_size(L):
    st, h = _create(L, 2, 2, 2, 128, 0)
    b = ctypes.c_size_t()
    assert L.lib().cgtp_workspace_size(h, 2000, 105730, ctypes.byref(b)) == L.CGTP_OK
    a = lambda v: (v + 255) // 256 * 256
    assert b.value == a(4 * 2001) + 2 * a(4 * 105730) + 2 * a(4 * 32 * 2000) + 2 * a(4 * 2000) + a(8 * 105730 * 2 * 9)
    assert L.lib().cgtp_workspace_size(h, -1, 5, ctypes.byref(b)) == L.CGTP_ERR_INVALID_ARG
    assert L.lib().cgtp_workspace_size(h, 5, 5, None) == L.CGTP_ERR_INVALID_ARG
    L.lib().cgtp_plan_destroy(h)


def test_calls_reject_bad_arguments_without_a_gpu(L):
    # every check below returns before any HIP call
    lib = L.lib()
    st, h = _create(L, 2, 2, 2, 128, 0)
    fake = ctypes.c_void_p(4096)       # never dereferenced: the checks fail first
    odd = ctypes.c_void_p(4096 + 4)    # not 8-byte aligned
    ws = ctypes.c_void_p(1 << 20)
    big = 1 << 30
    # null plan
    assert lib.cgtp_sh_fwd(None, 10, fake, fake, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_conv_fwd(None, 4, 4, fake, fake, fake, fake, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    # negative / oversized counts
    assert lib.cgtp_sh_fwd(h, -1, fake, fake, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_graph_prepare(h, -1, 4, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_graph_prepare(h, 4, 1 << 31, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    # missing graph arrays
    assert lib.cgtp_conv_fwd(h, 4, 4, None, fake, fake, fake, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, None, fake, fake, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    # workspace missing or too small
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, fake, fake, fake, fake, fake, None, big, None) == L.CGTP_ERR_WORKSPACE
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, fake, fake, fake, fake, fake, ws, 16, None) == L.CGTP_ERR_WORKSPACE
    assert lib.cgtp_conv_bwd(h, 4, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake, ws, 16,
                             None) == L.CGTP_ERR_WORKSPACE
    # misaligned channel arrays
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, fake, odd, fake, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, fake, fake, fake, odd, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_conv_bwd(h, 4, 4, fake, fake, fake, fake, fake, fake, odd, None, None, ws, big,
                             None) == L.CGTP_ERR_INVALID_ARG
    # missing inputs
    assert lib.cgtp_conv_fwd(h, 4, 4, fake, fake, None, fake, fake, fake, ws, big, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_conv_bwd(h, 4, 4, fake, fake, fake, fake, fake, None, fake, None, None, ws, big,
                             None) == L.CGTP_ERR_INVALID_ARG
    # nothing requested / nothing to do: OK without a launch
    assert lib.cgtp_conv_bwd(h, 4, 4, fake, fake, fake, fake, fake, fake, None, None, None, ws, big,
                             None) == L.CGTP_OK
    assert lib.cgtp_sh_fwd(h, 0, None, None, None) == L.CGTP_OK
    lib.cgtp_plan_destroy(h)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from clebsch_gordan_tensor_cgtp_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libcgtp.so not found"):
        _lib.lib()
