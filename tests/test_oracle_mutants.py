"""Planted mistakes in the CPU reference must be caught by its pins.

Each mutant is a copy of ``oracle/sgemm_ref.c`` (or ``oracle/conv_ref.c``)
with one plausible mistake
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

# Mistakes planted in oracle/conv_ref.c, caught by the convolution pins.
CONV_MUTANTS = [
    ("conv_pad_sign", "oh * sh - ph + r,\n", "oh * sh + ph + r,\n"),
    ("conv_swap_strides", "ow * sw - pw + s);\n                                    const double p",
     "ow * sh - pw + s);\n                                    const double p"),
    ("conv_swap_r_s", "const int c = k / (R * S), r = (k / S) % R, s = k % S;",
     "const int c = k / (R * S), s = (k / R) % S, r = k % R;"),
    ("conv_tap_bound", "if (ih < 0 || ih >= H || iw < 0 || iw >= W)",
     "if (ih < 0 || ih > H || iw < 0 || iw >= W)"),
    ("conv_channel_stride", "X[(((size_t)b * C + c) * H + ih) * W + iw]",
     "X[(((size_t)c * C + b) * H + ih) * W + iw]"),
    ("conv_output_order", "const size_t n0 = ((size_t)b * OH + oh) * OW;",
     "const size_t n0 = ((size_t)oh * OH + b) * OW;"),
    ("conv_drop_last_tap", "for (int k = 0; k < K; ++k) {\n                                const int c",
     "for (int k = 0; k + 1 < K; ++k) {\n                                const int c"),
    ("conv_skip_padding_products", "const double p = w * x;",
     "const double p = x != 0.0 ? w * x : 0.0;"),
    ("conv_drop_beta", "v = (alpha != 0.0) ? v + beta * (double)(*y) : beta * (double)(*y);",
     "v = (alpha != 0.0) ? v : beta * (double)(*y);"),
    ("conv_out_size_ceil", "return (in + 2 * pad - k) / stride + 1;",
     "return (in + 2 * pad - k + stride - 1) / stride + 1;"),
    ("im2col_transposed_tap", "const size_t k = ((size_t)c * R + r) * S + s;",
     "const size_t k = ((size_t)c * S + s) * R + r;"),
    ("im2col_pad_sign", "brow[n] = tap(X, C, H, W, b, c, oh * sh - ph + r, ow * sw - pw + s);",
     "brow[n] = tap(X, C, H, W, b, c, oh * sh - ph + r, ow * sw + pw + s);"),
    ("absdot_conv_signed", "mag[ow] = mag[ow] + fabs(p);", "mag[ow] = mag[ow] + p;"),
]

RUNNER = r'''
import sys
sys.path.insert(0, %(root)r)
import oracle
from tests import %(pins)s as pins
lib = oracle.load(%(lib)r)
caught = []
for pin in pins.ALL_PINS:
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
    _run_pins(lib, "oracle_pins", name)


def _run_pins(lib, pins, name):
    proc = subprocess.run([sys.executable, "-c",
                           RUNNER % {"root": ROOT, "lib": lib, "pins": pins}],
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, OMP_NUM_THREADS="2"))
    caught = proc.stdout.strip()
    # A crash from an out-of-range index also counts as caught.
    assert proc.returncode != 0 or caught, "no pin caught mutant %s" % name


@pytest.mark.parametrize("name,old,new", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_conv_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.CONV_SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    mutated = tmp_path / "mutant_conv.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(oracle.SOURCE, lib, conv_source=str(mutated))
    _run_pins(lib, "oracle_conv_pins", name)
