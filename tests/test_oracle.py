"""The CPU reference against its pins (closed forms, the page-3 worked
example, integer brute force, float64 library products, conventions)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_thread_count_does_not_change_bits(tmp_path):
    """Rows are split across threads, never k: one thread and many give the same bits."""
    A = workloads.uniform(97, 301, 5)
    B = workloads.uniform(301, 211, 6)
    np.save(tmp_path / "A.npy", A)
    np.save(tmp_path / "B.npy", B)
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r); import oracle;"
        "A=np.load(%r); B=np.load(%r); out,_=oracle.sgemm(A,B,None,1.25,0.0);"
        "np.save(%r, out)"
    )
    outs = []
    for threads in (1, 5):
        dst = str(tmp_path / ("out%d.npy" % threads))
        env = dict(os.environ, OMP_NUM_THREADS=str(threads))
        subprocess.run([sys.executable, "-c", code % (os.path.dirname(os.path.dirname(__file__)),
                                                       str(tmp_path / "A.npy"), str(tmp_path / "B.npy"), dst)],
                       check=True, env=env)
        outs.append(np.load(dst))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_points_agree_with_full_product(oracle_lib):
    """The two reference entry points (row-accumulated and per element) agree bit for bit."""
    A = workloads.uniform(33, 70, 90)
    B = workloads.uniform(70, 45, 91)
    C = workloads.uniform(33, 45, 92)
    full, t = oracle.sgemm(A, B, C, 0.75, -0.25, lib=oracle_lib)
    rows, cols = np.nonzero(np.ones((33, 45)))
    pts, tp = oracle.sgemm_points(A, B, C, 0.75, -0.25, rows, cols, lib=oracle_lib)
    assert np.array_equal(pts.view(np.uint32), full[rows, cols].view(np.uint32))
    assert np.array_equal(tp, t[rows, cols])


def test_tolerance_form():
    """At alpha = 1, beta = 0 the bound is 1e-5 * sum|a*b| + 1e-6."""
    t = np.array([0.0, 1.0, 1000.0])
    assert np.allclose(oracle.tolerance(1.0, 0.0, t, None), [1e-6, 1.1e-5, 1.0000e-2 + 1e-6])
    c = np.array([2.0, -2.0, 0.0])
    assert np.allclose(oracle.tolerance(-1.5, 0.5, t, c), 1e-5 * (1.5 * t + 0.5 * np.abs(c)) + 1e-6)
