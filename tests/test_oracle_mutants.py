"""Planted mistakes in the CPU reference must be caught by its pins.

Each mutant is a copy of ``oracle/sgemm_ref.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, a lost leading
dimension, float accumulation).  The copy is compiled into a temporary
library and the pins run against it in a child process (a wrong index may
read past an array, so the child keeps that away from the test runner).
The real reference is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in the reference, replacement)
MUTANTS = [
    ("drop_first_k", "for (int k = 0; k < K; ++k) {\n                        const double a",
     "for (int k = 1; k < K; ++k) {\n                        const double a"),
    ("subtract_products", "acc[j] = acc[j] + p;", "acc[j] = acc[j] - p;"),
    ("transpose_A", "(double)A[(size_t)i * lda + k]", "(double)A[(size_t)k * lda + i]"),
    ("transpose_B", "const double p = a * (double)brow[j];",
     "const double p = a * (double)B[(size_t)j * ldb + k];"),
    ("ignore_lda", "(double)A[(size_t)i * lda + k]", "(double)A[(size_t)i * K + k]"),
    ("ignore_ldb", "const float *brow = B + (size_t)k * ldb;", "const float *brow = B + (size_t)k * N;"),
    ("ignore_ldc", "float *crow = C + (size_t)i * ldc;", "float *crow = C + (size_t)i * N;"),
    ("drop_beta_term", "r = (alpha != 0.0) ? r + beta * (double)(*c) : beta * (double)(*c);",
     "r = (alpha != 0.0) ? r : beta * (double)(*c);"),
    ("swap_alpha_beta", "r = alpha * s;", "r = beta * s;"),
    ("beta_zero_reads_C", "    if (beta != 0.0)\n        r = (alpha",
     "    if (1)\n        r = (alpha"),
    ("float_accumulator", "const double p = a * (double)brow[j];\n                            acc[j] = acc[j] + p;",
     "const double p = a * (double)brow[j];\n                            acc[j] = (float)(acc[j] + p);"),
    ("points_transpose_B", "(double)B[(size_t)k * ldb + j]", "(double)B[(size_t)j * ldb + k]"),
    ("points_drop_last_k", "for (int k = 0; k < K; ++k) {\n                const double prod",
     "for (int k = 0; k + 1 < K; ++k) {\n                const double prod"),
    ("absdot_signed", "mag[j] = mag[j] + fabs(p);", "mag[j] = mag[j] + p;"),
]

RUNNER = r'''
import sys
sys.path.insert(0, %(root)r)
import oracle
from tests import oracle_pins
lib = oracle.load(%(lib)r)
caught = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except AssertionError:
        caught.append(pin.__name__)
print(",".join(caught))
'''


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(mutated), lib)
    proc = subprocess.run([sys.executable, "-c", RUNNER % {"root": ROOT, "lib": lib}],
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, OMP_NUM_THREADS="2"))
    caught = proc.stdout.strip()
    # A crash from an out-of-range index also counts as caught.
    assert proc.returncode != 0 or caught, "no pin caught mutant %s" % name
