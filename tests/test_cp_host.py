"""Host-side checks of the CP calls of libcgtp.so: the data-free factor fit
(alternating least squares, run on the host) against the oracle's from the
same start, its errors and argument checks, and the CP workspace size.  No
GPU is needed."""
import ctypes

import numpy as np
import pytest


@pytest.fixture(scope="module")
def L():
    from clebsch_gordan_tensor_cgtp_amd import _lib
    _lib.lib()
    return _lib


def _start(rng, plan, R):
    return (rng.standard_normal((plan.dim_out, R)), rng.standard_normal((plan.dim_in, R)),
            rng.standard_normal((plan.dim_sh, R)))


@pytest.mark.parametrize("Ls,R,sweeps", [((1, 1, 1), 6, 25), ((2, 2, 2), 20, 25), ((2, 1, 3), 12, 10),
                                         ((3, 3, 3), 40, 5), ((1, 1, 1), 16, 60)])
def test_fit_matches_the_oracle_als(L, oracle, Ls, R, sweeps):
    """Same start, same sweep order and ridge: the factors agree with the
    oracle's to rounding (the two solve the normal equations differently)."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(*Ls, 8)
    rng = np.random.default_rng(R)
    A0, B0, C0 = _start(rng, plan, R)
    A, B, C, err = plan.cp_fit(A0, B0, C0, sweeps)
    rA, rB, rC, hist = oracle.cp_als(oracle.cp_tensor(*Ls), A0, B0, C0, sweeps)
    for g, r in ((A, rA), (B, rB), (C, rC)):
        np.testing.assert_allclose(g, r, rtol=1e-6, atol=1e-8 * np.abs(r).max())
    assert err == pytest.approx(hist[-1], rel=1e-6, abs=1e-12)


def test_fit_reaches_the_exact_rank(oracle):
    """At rank d1*d2 the fit is exact to ~1e-6 (the tensor has such a
    decomposition), and at rank 64 so is the degree-2 tensor."""
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    rng = np.random.default_rng(3)
    plan = Plan(1, 1, 1, 8)
    *_, err = plan.cp_fit(*_start(rng, plan, 16), sweeps=300)
    assert err < 1e-6
    plan2 = Plan(2, 2, 2, 8)
    A, B, C, err2 = plan2.cp_fit(*_start(rng, plan2, 64), sweeps=300)
    assert err2 < 1e-6
    M = oracle.cp_tensor(2, 2, 2)
    assert np.sqrt(oracle.cp_objective(M, A, B, C) / (M ** 2).sum()) == pytest.approx(err2, rel=1e-3, abs=1e-12)


def test_fit_arguments(L):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(1, 1, 1, 8)
    lib = L.lib()
    z = np.zeros((4, 3))
    p = ctypes.c_void_p(z.ctypes.data)
    assert lib.cgtp_cp_fit(None, 3, 1, 0.0, p, p, p, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_cp_fit(plan._h, 0, 1, 0.0, p, p, p, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_cp_fit(plan._h, 3, -1, 0.0, p, p, p, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_cp_fit(plan._h, 3, 1, -1.0, p, p, p, None) == L.CGTP_ERR_INVALID_ARG
    assert lib.cgtp_cp_fit(plan._h, 3, 1, 0.0, None, p, p, None) == L.CGTP_ERR_INVALID_ARG
    # all-zero factors: the normal matrix is singular without a ridge
    A, B, C = np.zeros((4, 3)), np.zeros((4, 3)), np.zeros((4, 3))
    dp = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.cgtp_cp_fit(plan._h, 3, 1, 0.0, dp(A), dp(B), dp(C), None) == L.CGTP_ERR_NUMERIC
    # zero sweeps leave the start and report its error
    rng = np.random.default_rng(0)
    A0, B0, C0 = rng.standard_normal((4, 2)), rng.standard_normal((4, 2)), rng.standard_normal((4, 2))
    A1, B1, C1, err = plan.cp_fit(A0, B0, C0, sweeps=0)
    np.testing.assert_array_equal(A1, A0)
    with pytest.raises(ValueError):
        plan.cp_fit(A0[:3], B0, C0, sweeps=1)


def test_cp_workspace_size(L):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 100)
    base = plan.workspace_size(1000, 5000)
    for R, RP in ((1, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
        got = plan.cp_workspace_size(R, 1000, 5000)
        # xb and ga: N*RP*C fp64 each; yc: E*RP fp64; dyc: E*2*RP fp64 (C > 64);
        # the fp64 grad_W of the backward's passes (E*C) beyond rank 32
        want = base + 2 * 1000 * RP * 100 * 8 + 5000 * RP * 8 + 5000 * 2 * RP * 8 + (5000 * 100 * 8 if RP > 32 else 0)
        assert want <= got <= want + 5 * 256, R
    b = ctypes.c_size_t()
    assert L.lib().cgtp_cp_workspace_size(plan._h, 65, 10, 10, ctypes.byref(b)) == L.CGTP_ERR_UNSUPPORTED
    assert L.lib().cgtp_cp_workspace_size(plan._h, 0, 10, 10, ctypes.byref(b)) == L.CGTP_ERR_INVALID_ARG


def test_cp_conv_rejects_bad_arguments_without_a_gpu(L):
    from clebsch_gordan_tensor_cgtp_amd.ops import Plan
    plan = Plan(2, 2, 2, 64)
    lib = L.lib()
    fake, odd, ws = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8), ctypes.c_void_p(1 << 20)
    big = 1 << 34
    fwd = lambda R, x=fake, out=fake, wsb=big: lib.cgtp_cp_conv_fwd(plan._h, R, 4, 4, fake, fake, x, fake, fake,
                                                                     fake, fake, fake, out, ws, wsb, None)
    assert fwd(0) == L.CGTP_ERR_INVALID_ARG
    assert fwd(65) == L.CGTP_ERR_UNSUPPORTED
    assert fwd(8, wsb=16) == L.CGTP_ERR_WORKSPACE
    assert fwd(8, x=odd) == L.CGTP_ERR_INVALID_ARG
    assert fwd(8, out=None) == L.CGTP_ERR_INVALID_ARG
    bwd = lambda *o: lib.cgtp_cp_conv_bwd(plan._h, 8, 4, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                          *o, ws, big, None)
    assert bwd(None, None, None) == L.CGTP_OK
    assert bwd(odd, None, None) == L.CGTP_ERR_INVALID_ARG
