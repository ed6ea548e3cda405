"""Builds libcgtp.so (HIP, gfx950) in-tree.

Usage: ``python -m clebsch_gordan_tensor_cgtp_amd.build`` or
``python clebsch_gordan_tensor_cgtp_amd/build.py``.  Always recompiles.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcgtp.so")
BUILD = os.path.join(ROOT, "_build")

# the degree-3 kernels are split by lane geometry, one translation unit each,
# so the slowest compiles run in parallel (longest first)
SOURCES = ["cgtp_kernels_l3_c64_bwd.hip", "cgtp_kernels_l3_c64_bwd2.hip", "cgtp_kernels_l3_c128.hip", "cgtp_kernels_l3_c64.hip", "cgtp_kernels_l3_c32.hip",
           "cgtp_kernels_l3_c16.hip", "cgtp_kernels_l3_c8.hip", "cgtp_kernels_l2_wide.hip", "cgtp_kernels_l2.hip",
           "cgtp_kernels_l1.hip", "cgtp_cp.hip", "cgtp_mix.hip", "cgtp_registry.hip", "cgtp_graph.hip", "cgtp_forces.hip",
           "cgtp_cp_fit.cpp", "cgtp_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 ops stay off (the arithmetic is fp64 anyway)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if os.environ.get("CGTP_RESOURCE_USAGE") else []
    cmd = [HIPCC] + COMMON + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build_lib(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build_lib(verbose=True)
    sys.exit(0)
