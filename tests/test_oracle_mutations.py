"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, index or operand, a dropped projection), builds it into
a temporary library, and runs the oracle's pin tests against it in a
subprocess (CGTP_ORACLE_LIB points the oracle package at the copy).  The
case passes when at least one pin fails.  The committed oracle is never
modified, and nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "cgtp_oracle.c")
PINS = ["tests/test_oracle_cg.py", "tests/test_oracle_sh.py", "tests/test_oracle_conv.py",
        "tests/test_oracle_forces.py", "tests/test_oracle_cp.py"]

# (name, text in the oracle source, replacement): each text occurs exactly once
MUTATIONS = [
    ("racah sum sign dropped", "sum += (k & 1) ? -term : term;", "sum += term;"),
    ("CG prefactor 2J+1 -> 2J", "double pre = sqrt((2.0 * J + 1.0) *", "double pre = sqrt((2.0 * J) *"),
    ("basis: (-1)^m dropped for m > 0", "if (mu == m) *re = sgn * s;", "if (mu == m) *re = s;"),
    ("basis: conjugation dropped", "ci = -ci; /* conjugate */", "ci = ci; /* conjugate */"),
    ("real part taken for odd paths", "double v = odd ? im[i] : re[i];", "double v = re[i];"),
    ("SH l=1 components swapped", "o[1] = c1 * y;", "o[1] = c1 * x;"),
    ("SH l=2 sign", "o[8] = 0.25 * sqrt(15.0 / pi) * (x * x - y * y);",
     "o[8] = 0.25 * sqrt(15.0 / pi) * (y * y - x * x);"),
    ("SH l=3 coefficient", "o[12] = 0.25 * sqrt(7.0 / pi) * (5.0 * z * z * z - 3.0 * z);",
     "o[12] = 0.25 * sqrt(7.0 / pi) * (5.0 * z * z * z - 2.0 * z);"),
    ("forward: weight dropped", "o[(l3 * l3 + l3 + m3) * C + u] += w * c * xv * yv;",
     "o[(l3 * l3 + l3 + m3) * C + u] += c * xv * yv;"),
    ("forward: m1 index flipped",
     "double xv = x[(j * Din + l1 * l1 + l1 + m1) * C + u];\n                                double yv = Y[e * Dsh + l2 * l2 + l2 + m2];\n                                o[",
     "double xv = x[(j * Din + l1 * l1 + l1 - m1) * C + u];\n                                double yv = Y[e * Dsh + l2 * l2 + l2 + m2];\n                                o["),
    ("backward: weight dropped in grad_Y",
     "acc += c * xv * yv * gv;\n                                if (dY) dY[e * Dsh + l2 * l2 + l2 + m2] += w * c * xv * gv;",
     "acc += c * xv * yv * gv;\n                                if (dY) dY[e * Dsh + l2 * l2 + l2 + m2] += c * xv * gv;"),
    ("backward: grad_W without grad_out",
     "acc += c * xv * yv * gv;\n                                if (dY) dY",
     "acc += c * xv * yv;\n                                if (dY) dY"),
    ("backward: grad_x scattered to the receiver", "mine[(j * Din + l1 * l1 + l1 + m1) * C + u] += w * c * yv * gv;",
     "mine[(i * Din + l1 * l1 + l1 + m1) * C + u] += w * c * yv * gv;"),
    ("transpose: receivers walked backwards",
     "    for (int64_t i = 0; i < N; ++i)\n        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {\n            int64_t k = cursor[src[e]]++;",
     "    for (int64_t i = N - 1; i >= 0; --i)\n        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {\n            int64_t k = cursor[src[e]]++;"),
    ("SH backward: tangential projection dropped", "dr[3 * e + 0] = (gx - x * ug) / n;", "dr[3 * e + 0] = gx / n;"),
    ("SH backward: wrong l=2 derivative", "gz += w[6] * 6.0 * b * z;", "gz += w[6] * 3.0 * b * z;"),
    ("SH backward: wrong l=3 derivative", "gx += w[15] * 3.0 * a * (x * x - y * y);",
     "gx += w[15] * 3.0 * a * (x * x + y * y);"),
    ("node gradient: receiver sign", "dpos[3 * i + a] -= dr[3 * e + a];", "dpos[3 * i + a] += dr[3 * e + a];"),
    ("double backward: ggY term dropped from d_out",
     "c * (ORC_GX(a) * ORC_Y(b) * ORC_W + ORC_X(a) * ORC_GY(b) * ORC_W +",
     "c * (ORC_GX(a) * ORC_Y(b) * ORC_W + 0.0 * ORC_GY(b) * ORC_W +"),
    ("double backward: weight and its cotangent swapped in d_Y",
     "if (dY) dY[e * Dsh + b] += c * (ORC_GX(a) * ORC_W + ORC_X(a) * ORC_GW) * ORC_G(k3);",
     "if (dY) dY[e * Dsh + b] += c * (ORC_GX(a) * ORC_GW + ORC_X(a) * ORC_W) * ORC_G(k3);"),
    ("double backward: d_x without the ggW term",
     "c * (ORC_GY(b) * ORC_W + ORC_Y(b) * ORC_GW) * ORC_G(k3);", "c * (ORC_GY(b) * ORC_W) * ORC_G(k3);"),
    ("CP forward: C^T y factor dropped", "for (int r = 0; r < R; ++r) z += A[c * R + r] * s[r] * t[r];",
     "for (int r = 0; r < R; ++r) z += A[c * R + r] * s[r];"),
    ("CP backward: B^T x used in g_x", "for (int r = 0; r < R; ++r) v += B[a * R + r] * ga[r] * t[r];",
     "for (int r = 0; r < R; ++r) v += B[a * R + r] * ga[r] * s[r];"),
    ("CP backward: edge weight dropped in g_y", "dY[e * d2 + b] += w * v;", "dY[e * d2 + b] += v;"),
    ("per-path outputs: m3 flipped", "op[(o[p] + l3 + m3) * C + u] += w * c *", "op[(o[p] + l3 - m3) * C + u] += w * c *"),
    ("per-path backward: the summed slot read", "const double gv = G[(i * Dmid + o[p] + l3 + m3) * C + u];",
     "const double gv = G[(i * Dmid + l3 * l3 + l3 + m3) * C + u];"),
]


def test_mutations_apply_exactly_once():
    text = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert text.count(old) == 1, name
        assert old != new, name


def test_unmutated_oracle_passes_the_pins_in_the_harness(tmp_path):
    """Control: the harness itself reports success for the committed source."""
    assert _run_pins(tmp_path, open(SRC).read()) == 0


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    text = open(SRC).read()
    assert _run_pins(tmp_path, text.replace(old, new)) != 0, f"no pin caught: {name}"


def _run_pins(tmp_path, source):
    sys.path.insert(0, ROOT)
    from oracle.build import build_oracle
    src = tmp_path / "oracle_copy.c"
    src.write_text(source)
    lib = build_oracle(src=str(src), lib=str(tmp_path / "liboracle_copy.so"))
    env = dict(os.environ, CGTP_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode
