"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte
accounting behind the roofline, and the PMC-summary lookup."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_algorithmic_bytes_per_edge_and_node():
    # L = 2, C = 128, P = 15, D = 9: forward 7720 B per edge + 9220 B per node,
    # backward 15440 B per edge + 13828 B per node (each tensor once)
    N, E = 2000, 105730
    ab = bench.algorithmic_bytes(N, E, 15, 128, 9, 9, 9)
    assert ab["fwd"] == E * 7720 + N * 9220 == 834_675_600
    assert ab["bwd"] == E * 15440 + N * 13828 == 1_660_127_200
    # per-edge parts scale with E only, per-node parts with N only
    ab2 = bench.algorithmic_bytes(2 * N, 3 * E, 15, 128, 9, 9, 9)
    assert ab2["fwd"] == 3 * E * 7720 + 2 * N * 9220
    assert ab2["bwd"] == 3 * E * 15440 + 2 * N * 13828


def test_traffic_is_read_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    assert len(sha) == 16
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = tmp_path / "profiles" / "pmc_conv_bwd_layer.txt"
    assert bench.read_traffic("conv_bwd", "layer") is None  # no summary
    f.write_text("# header\nhbm_bytes_per_launch = 123456\nkernel_source_sha = 0000000000000000\n")
    assert bench.read_traffic("conv_bwd", "layer") is None  # other sources
    f.write_text(f"hbm_bytes_per_launch = 123456\nkernel_source_sha = {sha}\n")
    assert bench.read_traffic("conv_bwd", "layer") == pytest.approx(123456.0)


def test_step_kernel_names_pick_the_step_kernels():
    """The summaries find the step's forward and backward among every
    instantiation of the two templates by their full signature: the plain
    (or SUB) form with DBL, MID and FSH false, either PS."""
    step = ["void cgtp::k_conv_fwd<2, 64, 2, false, false, false, false>(cgtp::FwdArgs)",
            "void cgtp::k_conv_bwd<2, 64, 2, false, false, false, false, false>(cgtp::BwdArgs)",
            "void cgtp::k_conv_bwd<3, 64, 1, false, false, false, false, true>(cgtp::BwdArgs)"]
    other = ["void cgtp::k_conv_fwd<2, 64, 2, true, true, false, false>(cgtp::FwdArgs)",       # double backward
             "void cgtp::k_conv_fwd<3, 64, 1, true, true, false, true>(cgtp::FwdArgs)",
             "void cgtp::k_conv_fwd<2, 64, 2, false, false, true, false>(cgtp::FwdArgs)",      # fused SH
             "void cgtp::k_conv_bwd<2, 64, 2, true, true, false, false, false>(cgtp::BwdArgs)",
             "void cgtp::k_conv_bwd<2, 64, 2, true, false, true, false, false>(cgtp::BwdArgs)",  # per-path
             "void cgtp::k_conv_bwd<3, 64, 1, false, false, false, true, true>(cgtp::BwdArgs)"]  # fused SH
    for name in step:
        kern = "conv_fwd" if "k_conv_fwd" in name else "conv_bwd"
        assert bench.re.search(bench.STEP_KERNEL[kern], name), name
    for name in other:
        assert not any(bench.re.search(p, name) for p in bench.STEP_KERNEL.values()), name
