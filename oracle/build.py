"""Builds the fp64 CPU oracle (test infrastructure) with gcc.

Usage: ``python oracle/build.py``.  Produces ``oracle/liboracle.so``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cgtp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile ``src`` (default ``cgtp_oracle.c``) into ``lib`` (default
    ``liboracle.so``); always recompiles."""
    tmp = lib + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build_oracle(verbose=True)
    sys.exit(0)
