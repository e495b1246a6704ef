"""Planted mistakes in the CPU oracle must fail the pins.

Each mutant is a copy of the oracle's C source with one plausible slip, built
with gcc into a temporary directory and loaded in a child pytest run through the
M3REF_LIB override.  The shipped oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "m3ref.c")

MUTANTS = {
    "delayed write indexed at t": [(
        "Hs[i] = alpha * Hs[i] + beta * Vp[i];", "Hs[i] = alpha * Hs[i] + beta * Vc[i];")],
    "rotation clockwise": [(
        "r0[p] = c * u - s * v;\n            r1[p] = s * u + c * v;",
        "r0[p] = c * u + s * v;\n            r1[p] = -s * u + c * v;")],
    "current write rotated too": [(
        "if (theta) rotate_pairs(Hs, N, P, theta + tok * (N / 2));\n"
        "                    for (size_t i = 0; i < NP; ++i) Hs[i] += gamma * Vc[i];",
        "for (size_t i = 0; i < NP; ++i) Hs[i] += gamma * Vc[i];\n"
        "                    if (theta) rotate_pairs(Hs, N, P, theta + tok * (N / 2));")],
    "previous write not rotated": [(
        "Hs[i] = alpha * Hs[i] + beta * Vp[i];\n"
        "                    if (theta) rotate_pairs(Hs, N, P, theta + tok * (N / 2));",
        "Hs[i] = alpha * Hs[i];\n"
        "                    if (theta) rotate_pairs(Hs, N, P, theta + tok * (N / 2));\n"
        "                    for (size_t i = 0; i < NP; ++i) Hs[i] += beta * Vp[i];")],
    "beta without alpha": [(
        "const double beta = (1.0 - lm) * d * alpha;", "const double beta = (1.0 - lm) * d;")],
    "endpoint weights swapped": [(
        "const double gamma = lm * d;", "const double gamma = (1.0 - lm) * d;")],
    "pairs are halves": [(
        "double* r0 = M + (size_t)(2 * k) * P;\n        double* r1 = M + (size_t)(2 * k + 1) * P;",
        "double* r0 = M + (size_t)k * P;\n        double* r1 = M + (size_t)(k + N / 2) * P;")],
    "MIMO operand mismatched": [(
        "acc += Bm[(size_t)r * N + n] * Xm[(size_t)r * P + p];",
        "acc += Bm[(size_t)r * N + n] * Xm[(size_t)((r + 1) % R) * P + p];")],
    "carried write dropped": [(
        "if (B_prev)\n                    mimo_write", "if (0)\n                    mimo_write")],
    "decay sign flipped": [(
        "const double alpha = exp(d * A[h]);", "const double alpha = exp(-d * A[h]);")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_pins(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor missing for {name!r}"
        src = src.replace(old, new)
    c = tmp_path / "m.c"
    c.write_text(src)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", str(c), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, M3REF_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert r.returncode != 0, f"mutant {name!r} passed every pin:\n{r.stdout[-2000:]}"
