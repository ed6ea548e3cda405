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
    assert len(names) == 23
    for n in names:
        assert hasattr(L.lib(), n), n
        assert n in L.SIGNATURES, n


def test_binding_argument_counts_match_header(L):
    """Every ctypes signature takes as many arguments as its declaration."""
    text = open(os.path.join(ROOT, "include", "cgtp.h")).read()
    for name, params in re.findall(r"^(?:cgtp_status_t|const char\*)\s+(cgtp_\w+)\(([^)]*)\);", text, re.M):
        n = len([p for p in params.split(",") if p.strip()])
        assert len(L.SIGNATURES[name][1]) == n, name


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
    assert _create(L, 2, 2, 2, 128, 16)[0] == L.CGTP_ERR_INVALID_ARG     # unknown flag bit
    assert _create(L, 4, 4, 4, 16, 0)[0] == L.CGTP_ERR_UNSUPPORTED
    assert _create(L, 1, 4, 1, 16, 0)[0] == L.CGTP_ERR_UNSUPPORTED
    assert _create(L, 2, 2, 2, 129, 0)[0] == L.CGTP_ERR_UNSUPPORTED     # more than 128 channels
    # every degree triple up to 3 and every channel count from 1 to 128
    for (a, b, c) in ((0, 0, 0), (1, 1, 1), (2, 3, 2), (3, 0, 3), (0, 2, 2), (3, 3, 3)):
        for C in (1, 7, 8, 24, 64, 65, 96, 127, 128):
            for flags in (0, L.CGTP_FLAG_VALIDATE, L.CGTP_FLAG_LOCALITY, L.CGTP_FLAG_SHARED_WEIGHTS,
                          L.CGTP_FLAG_PATH_OUTPUTS):
                st, h = _create(L, a, b, c, C, flags)
                assert st == L.CGTP_OK, (a, b, c, C, flags)
                assert L.lib().cgtp_plan_destroy(h) == L.CGTP_OK
    assert L.lib().cgtp_plan_destroy(None) == L.CGTP_OK


TRIPLES = [(a, b, c) for a in range(4) for b in range(4) for c in range(4)]


@pytest.mark.parametrize("a,b,c", TRIPLES)
def test_plan_paths_and_tables_match_oracle(L, oracle, a, b, c):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(a, b, c, 8)
    assert plan.paths == [tuple(int(v) for v in p) for p in oracle.paths(a, b, c)]
    assert (plan.dim_in, plan.dim_sh, plan.dim_out) == ((a + 1) ** 2, (b + 1) ** 2, (c + 1) ** 2)
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
    from tests.layout import ws_sections
    st, h = _create(L, 2, 2, 2, 128, 0)
    b = ctypes.c_size_t()
    for N, E in ((2000, 105730), (0, 0), (1, 0), (13, 5), (50000, 2616668)):
        assert L.lib().cgtp_workspace_size(h, N, E, ctypes.byref(b)) == L.CGTP_OK
        assert b.value == ws_sections(N, E)["total"]
        assert b.value <= 16 * max(E, 1) + 170 * max(N, 1) + 16384 + 15 * 256  # the header's estimate, plus alignment
    assert L.lib().cgtp_workspace_size(h, -1, 5, ctypes.byref(b)) == L.CGTP_ERR_INVALID_ARG
    assert L.lib().cgtp_workspace_size(h, 5, 5, None) == L.CGTP_ERR_INVALID_ARG
    L.lib().cgtp_plan_destroy(h)


def test_calls_reject_bad_arguments_without_a_gpu(L):
    # every check below returns before any HIP call
    lib = L.lib()
    st, h = _create(L, 2, 2, 2, 128, 0)
    fake = ctypes.c_void_p(4096)       # never dereferenced: the checks fail first
    odd = ctypes.c_void_p(4096 + 8)    # not 16-byte aligned
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
    # double backward: (x, Y, W, grad_out, gg_x, gg_Y, gg_W, dd_x, dd_Y, dd_W, dd_out)
    dbl = lambda *p, ws_=ws, n=big: lib.cgtp_conv_bwd_bwd(h, 4, 4, fake, fake, *p, ws_, n, None)
    assert dbl(fake, fake, fake, fake, None, None, None, fake, None, None, None, ws_=ws, n=16) == L.CGTP_ERR_WORKSPACE
    assert dbl(None, fake, fake, fake, None, None, None, fake, None, None, None) == L.CGTP_ERR_INVALID_ARG
    assert dbl(fake, fake, fake, None, None, None, None, fake, None, None, None) == L.CGTP_ERR_INVALID_ARG
    assert dbl(fake, fake, fake, fake, odd, None, None, fake, None, None, None) == L.CGTP_ERR_INVALID_ARG
    assert dbl(fake, fake, fake, fake, None, None, None, None, None, None, odd) == L.CGTP_ERR_INVALID_ARG
    assert dbl(fake, fake, fake, fake, fake, fake, fake, None, None, None, None) == L.CGTP_OK
    # fused-SH forward (x, r, W, out) and backward (x, r, W, grad_out, grad_x, grad_W, grad_r)
    fsh = lambda *p, ws_=ws, n=big: lib.cgtp_conv_fwd_sh(h, 4, 4, fake, fake, *p, ws_, n, None)
    bsh = lambda *p, ws_=ws, n=big: lib.cgtp_conv_bwd_sh(h, 4, 4, fake, fake, *p, ws_, n, None)
    assert fsh(fake, fake, fake, fake, ws_=None) == L.CGTP_ERR_WORKSPACE
    assert fsh(fake, None, fake, fake) == L.CGTP_ERR_INVALID_ARG
    assert fsh(fake, odd, fake, fake) == L.CGTP_ERR_INVALID_ARG
    assert fsh(fake, fake, fake, None) == L.CGTP_ERR_INVALID_ARG
    assert bsh(fake, fake, fake, fake, None, None, None) == L.CGTP_OK
    assert bsh(fake, None, fake, fake, None, None, fake) == L.CGTP_ERR_INVALID_ARG
    assert bsh(fake, fake, fake, fake, None, None, odd) == L.CGTP_ERR_INVALID_ARG
    assert bsh(fake, fake, fake, fake, None, None, fake, n=16) == L.CGTP_ERR_WORKSPACE
    lib.cgtp_plan_destroy(h)
    # per-path-output plans have no fused-SH form
    st, hm = _create(L, 2, 2, 2, 64, L.CGTP_FLAG_PATH_OUTPUTS)
    assert st == L.CGTP_OK
    assert lib.cgtp_conv_fwd_sh(hm, 4, 4, fake, fake, fake, fake, fake, fake, ws, big, None) == L.CGTP_ERR_UNSUPPORTED
    assert lib.cgtp_conv_bwd_sh(hm, 4, 4, fake, fake, fake, fake, fake, fake, fake, None, fake, ws, big,
                                None) == L.CGTP_ERR_UNSUPPORTED
    lib.cgtp_plan_destroy(hm)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from clebsch_gordan_tensor_cgtp_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libcgtp.so not found"):
        _lib.lib()


def test_noalloc_backward_rejects_graphs_beyond_its_scratch(L):
    """The allocation-free backward refuses a graph whose workspace exceeds
    its 64 MiB static scratch, before any HIP call."""
    lib = L.lib()
    st, h = _create(L, 2, 2, 2, 128, 0)
    fake = ctypes.c_void_p(4096)
    b = ctypes.c_size_t()
    lib.cgtp_workspace_size(h, 100000, 5_000_000, ctypes.byref(b))
    assert b.value > 64 << 20
    assert lib.cgtp_conv_bwd_noalloc(h, 100000, 5_000_000, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                     None) == L.CGTP_ERR_WORKSPACE
    assert lib.cgtp_conv_bwd_noalloc(None, 10, 10, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                     None) == L.CGTP_ERR_INVALID_ARG
    lib.cgtp_plan_destroy(h)


def test_path_outputs_plan_reports_the_per_path_width(L):
    """With per-path outputs dim_out is the sum over the paths of 2*l3+1."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    for (a, b, c), want in (((1, 1, 1), 11), ((2, 2, 2), 51), ((3, 3, 3), 156), ((2, 1, 3), None)):
        plan = Plan(a, b, c, 16, path_outputs=True)
        rows = sum(2 * l3 + 1 for (_, _, l3) in plan.paths)
        assert plan.dim_out == rows and (want is None or rows == want)
        assert plan.dim_z == (c + 1) ** 2


def test_path_mix_arguments_without_a_gpu(L):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64)
    lib = L.lib()
    fake, odd, ws = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8), ctypes.c_void_p(1 << 20)
    b = ctypes.c_size_t()
    assert lib.cgtp_path_mix_workspace_size(plan._h, 1000, 0, ctypes.byref(b)) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_path_mix_workspace_size(plan._h, 1000, 1025, ctypes.byref(b)) == L.CGTP_ERR_UNSUPPORTED
    assert lib.cgtp_path_mix_workspace_size(plan._h, 1000, 128, ctypes.byref(b)) == L.CGTP_OK
    # fp64 partials of the weight gradient's runs: 1 x 2 output tiles -> 512 runs wanted over the
    # 1000 x 51 (component, node) pairs -> runs of ceil(100 / 32) * 32 = 128 pairs; the 3, 6 and 6
    # paths of l3 = 0, 1, 2 take 8, 24 and 40 runs each: 408 runs of [64][128] doubles
    assert b.value == 8 * 408 * 64 * 128
    assert lib.cgtp_path_mix_workspace_size(plan._h, 2**31 - 1, 128, ctypes.byref(b)) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_path_mix_fwd(None, 10, 8, fake, fake, fake, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_path_mix_fwd(plan._h, 10, 8, odd, fake, fake, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_path_mix_fwd(plan._h, 10, 2000, fake, fake, fake, None) == L.CGTP_ERR_UNSUPPORTED
    assert lib.cgtp_path_mix_bwd(plan._h, 10, 8, fake, fake, fake, None, None, None, 0, None) == L.CGTP_OK
    assert lib.cgtp_path_mix_bwd(plan._h, 10, 8, fake, fake, fake, None, fake, ws, 16, None) == L.CGTP_ERR_WORKSPACE
    assert lib.cgtp_path_mix_bwd(plan._h, 10, 8, fake, fake, None, fake, None, None, 0, None) == L.CGTP_ERR_INVALID_ARG
