"""Pins of the CPU reference to facts outside itself.

Each pin is a plain function ``pin_xxx(lib)`` that raises AssertionError when
the reference loaded as ``lib`` disagrees with something the pages or the
mathematics fix: closed forms, the page-3 worked example, integer brute force
against numpy's exact int64 product, float64 library products, and the
alpha/beta/ld conventions.  ``tests/test_oracle.py`` runs them against the
real reference; ``tests/test_oracle_mutants.py`` runs them against copies of
the reference with a mistake planted in its source and checks that some pin
catches each mistake.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def pin_ones_closed_form(lib):
    """ones(M,K) @ ones(K,N) = K in every element, exactly; ld padding ignored."""
    for M, N, K, pad in [(3, 5, 7, 0), (17, 9, 33, 3), (1, 1, 1, 0), (4, 64, 129, 5)]:
        A = workloads._embed(np.ones((M, K), np.float32), K + pad, np.nan)
        B = workloads._embed(np.ones((K, N), np.float32), N + pad, np.nan)
        out, t = oracle.sgemm(A, B, lib=lib)
        assert np.array_equal(out, np.full((M, N), K, np.float32)), (M, N, K)
        assert np.array_equal(t, np.full((M, N), K, np.float64)), (M, N, K)


def pin_identity(lib):
    """I_K @ B = B bit for bit."""
    K, N = 23, 31
    A = np.eye(K, dtype=np.float32)
    B = workloads.uniform(K, N, 7)
    out, _ = oracle.sgemm(A, B, lib=lib)
    assert np.array_equal(_bits(out), _bits(B))


def pin_page3_constant_case(lib):
    """Page 3's demo: A = 1, B = 0.01 gives C = K * float(0.01) in every element."""
    for K, a, b, hexval, tol in _golden_rows("page3_constant_case.txt"):
        K = int(K)
        expect = np.array([int(hexval, 16)], np.uint32).view(np.float32)[0]
        A = np.full((8, K), np.float32(a), np.float32)
        B = np.full((K, 8), np.float32(b), np.float32)
        out, _ = oracle.sgemm(A, B, lib=lib)
        assert np.all(_bits(out) == np.uint32(int(hexval, 16))), out[0, 0]
        assert np.all(np.abs(out.astype(np.float64) - 10.24) <= float(tol))
        assert expect == np.float32(10.24)


def pin_cancellation_needs_fp64(lib):
    """a = [1e8, 1, -1e8], b = [1, 1, 1]: the double-accumulated sum is exactly 1."""
    for row in _golden_rows("cancellation.txt"):
        vals = [float(v) for v in row]
        A = np.array([vals[0:3]], np.float32)
        B = np.array(vals[3:6], np.float32).reshape(3, 1)
        out, t = oracle.sgemm(A, B, lib=lib)
        assert out[0, 0] == np.float32(vals[6]), out[0, 0]
        assert t[0, 0] == 2e8 + 1.0
        pts, _ = oracle.sgemm_points(A, B, None, 1.0, 0.0, np.array([0]), np.array([0]), lib=lib)
        assert pts[0] == np.float32(vals[6])


def pin_one_hot_rows_of_B(lib):
    """A = e_i e_k^T selects row k of B into row i of C; all other rows are 0."""
    M, N, K = 5, 9, 7
    B = workloads.uniform(K, N, 11)
    for i, k in [(0, 0), (4, 6), (2, 3), (3, 0)]:
        A = np.zeros((M, K), np.float32)
        A[i, k] = 1.0
        out, _ = oracle.sgemm(A, B, lib=lib)
        expect = np.zeros((M, N), np.float32)
        expect[i] = B[k]
        assert np.array_equal(_bits(out), _bits(expect)), (i, k)


def pin_one_hot_columns_of_A(lib):
    """B = e_k e_j^T selects column k of A into column j of C."""
    M, N, K = 6, 8, 5
    A = workloads.uniform(M, K, 12)
    for k, j in [(0, 0), (4, 7), (2, 5)]:
        B = np.zeros((K, N), np.float32)
        B[k, j] = 1.0
        out, _ = oracle.sgemm(A, B, lib=lib)
        expect = np.zeros((M, N), np.float32)
        expect[:, j] = A[:, k]
        assert np.array_equal(_bits(out), _bits(expect)), (k, j)


def pin_integer_brute_force(lib):
    """Every (M, N, K) in {1..6}^3 with integer data equals numpy's exact int64 product."""
    s = 0
    for M, N, K in itertools.product(range(1, 7), repeat=3):
        s += 1
        A = workloads.integers(M, K, 1000 + s)
        B = workloads.integers(K, N, 2000 + s)
        exact = A.astype(np.int64) @ B.astype(np.int64)
        out, t = oracle.sgemm(A, B, lib=lib)
        assert np.array_equal(out, exact.astype(np.float32)), (M, N, K)
        assert np.array_equal(t, (np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))).astype(np.float64))


def pin_alpha_beta_integer(lib):
    """alpha = 1.5, beta = 0.5 on integer data: exactly 1.5*(A@B) + 0.5*C (all dyadic)."""
    for M, N, K in [(7, 11, 13), (16, 3, 40), (1, 33, 2)]:
        A = workloads.integers(M, K, 31)
        B = workloads.integers(K, N, 32)
        C = workloads.integers(M, N, 33)
        exact = 1.5 * (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64) + 0.5 * C.astype(np.float64)
        out, _ = oracle.sgemm(A, B, C, alpha=1.5, beta=0.5, lib=lib)
        assert np.array_equal(out, exact.astype(np.float32)), (M, N, K)
        # the sign of alpha and beta matters
        exact2 = -2.0 * (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64) - 3.0 * C.astype(np.float64)
        out2, _ = oracle.sgemm(A, B, C, alpha=-2.0, beta=-3.0, lib=lib)
        assert np.array_equal(out2, exact2.astype(np.float32)), (M, N, K)


def pin_leading_dimensions(lib):
    """Padded rows (ld > cols) give the same result as packed rows; padding is never read."""
    M, N, K = 9, 13, 21
    A = workloads.integers(M, K, 41)
    B = workloads.integers(K, N, 42)
    C = workloads.integers(M, N, 43)
    ref, _ = oracle.sgemm(A, B, C, 1.0, 1.0, lib=lib)
    Ap = workloads._embed(A, K + 7, np.nan)
    Bp = workloads._embed(B, N + 3, np.nan)
    Cp = workloads._embed(C, N + 5, np.nan)
    out, _ = oracle.sgemm(Ap, Bp, Cp, 1.0, 1.0, lib=lib)
    assert np.array_equal(out, ref)
    # the padding of C's rows is left alone
    assert out.strides[0] == 4 * (N + 5)
    full = np.lib.stride_tricks.as_strided(out, shape=(M, N + 5), strides=out.strides)
    assert np.all(np.isnan(full[:, N:]))
    exact = (A.astype(np.int64) @ B.astype(np.int64) + C.astype(np.int64)).astype(np.float32)
    assert np.array_equal(out, exact)


def pin_random_vs_float64_library(lib):
    """Uniform data: the reference equals float32(numpy float64 product) to one ulp,
    mostly bit for bit, and its sum|a*b| matches |A| @ |B| in float64."""
    for M, N, K in [(37, 41, 129), (64, 3, 1000), (5, 70, 1)]:
        A = workloads.uniform(M, K, 51)
        B = workloads.uniform(K, N, 52)
        C = workloads.uniform(M, N, 53)
        ref64 = A.astype(np.float64) @ B.astype(np.float64)
        out, t = oracle.sgemm(A, B, C, 1.0, 0.0, lib=lib)
        lib32 = ref64.astype(np.float32)
        ulps = np.abs(_bits(out).astype(np.int64) - _bits(lib32).astype(np.int64))
        assert ulps.max() <= 1, ulps.max()
        assert np.mean(ulps == 0) > 0.99
        tref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.allclose(t, tref, rtol=1e-12, atol=0)
        # alpha/beta path against the float64 library product
        out2, _ = oracle.sgemm(A, B, C, 1.5, 0.5, lib=lib)
        want = (1.5 * ref64 + 0.5 * C.astype(np.float64)).astype(np.float32)
        ulps2 = np.abs(_bits(out2).astype(np.int64) - _bits(want).astype(np.int64))
        assert ulps2.max() <= 1


def pin_beta_zero_does_not_read_C(lib):
    """beta = 0: C is written, not read, so NaN in C does not reach the result."""
    A = workloads.integers(4, 6, 61)
    B = workloads.integers(6, 5, 62)
    C = np.full((4, 5), np.nan, np.float32)
    out, _ = oracle.sgemm(A, B, C, 2.0, 0.0, lib=lib)
    exact = (2 * (A.astype(np.int64) @ B.astype(np.int64))).astype(np.float32)
    assert np.array_equal(out, exact)
    rows, cols = np.nonzero(np.ones((4, 5)))
    pts, _ = oracle.sgemm_points(A, B, C, 2.0, 0.0, rows, cols, lib=lib)
    assert np.array_equal(pts, exact[rows, cols])


def pin_alpha_zero_and_empty_k(lib):
    """alpha = 0 or K = 0: C <- beta*C and A, B are not read (NaN operands)."""
    A = np.full((3, 4), np.nan, np.float32)
    B = np.full((4, 5), np.nan, np.float32)
    C = workloads.integers(3, 5, 71)
    out, _ = oracle.sgemm(A, B, C, 0.0, 0.5, lib=lib)
    assert np.array_equal(out, (0.5 * C.astype(np.float64)).astype(np.float32))
    out, _ = oracle.sgemm(A, B, C, 0.0, 0.0, lib=lib)
    assert np.array_equal(_bits(out), np.zeros((3, 5), np.uint32))
    A0 = np.zeros((3, 0), np.float32)
    B0 = np.zeros((0, 5), np.float32)
    out, t = oracle.sgemm(A0, B0, C, 1.0, -1.0, lib=lib)
    assert np.array_equal(out, -C)
    assert np.array_equal(t, np.zeros((3, 5)))


def pin_points_match_integer_product(lib):
    """The per-element path equals the exact int64 product at sampled points."""
    M, N, K = 40, 50, 60
    A = workloads.integers(M, K, 81)
    B = workloads.integers(K, N, 82)
    C = workloads.integers(M, N, 83)
    rng = np.random.default_rng(84)
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    exact = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64) * -1.5 + C.astype(np.float64) * 0.5
    pts, t = oracle.sgemm_points(A, B, C, -1.5, 0.5, rows, cols, lib=lib)
    assert np.array_equal(pts, exact[rows, cols].astype(np.float32))
    tref = (np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64)))[rows, cols]
    assert np.array_equal(t, tref.astype(np.float64))
    # padded leading dimensions on the point path too
    Ap = workloads._embed(A, K + 3, np.nan)
    Bp = workloads._embed(B, N + 1, np.nan)
    Cp = workloads._embed(C, N + 9, np.nan)
    pts2, _ = oracle.sgemm_points(Ap, Bp, Cp, -1.5, 0.5, rows, cols, lib=lib)
    assert np.array_equal(pts2, pts)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
