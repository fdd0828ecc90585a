"""CPU reference for SGEMM -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it, and it
imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``sgemm_ref.c`` and ``conv_ref.c`` (plain C, fp64
accumulation, one rounding at the end); this module only builds those files
with gcc and marshals numpy arrays into them.

What is computed, for row-major fp32 matrices::

    C[i, j] <- alpha * sum_k A[i, k] * B[k, j] + beta * C[i, j]

following the CPU reference loop of "matmul_opt.cu" (cnblogs post) and the
alpha/beta epilogue of the NVIDIA_SGEMM_PRACTICE README (kernel 1 section),
and the 2-D convolution (cross-correlation, NCHW input, zero padding) that
the UNIVERSAL_SGEMM_CUDA README's convolution-as-GEMM shapes stand for,
with its im2col lowering.  The GEMM functions are pinned by
``tests/test_oracle.py`` against closed forms, integer brute force and
float64 library products; the convolution functions by
``tests/test_oracle_conv.py`` against scipy's correlation, padded sliding
windows, 1x1 products and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sgemm_ref.c")
CONV_SOURCE = os.path.join(_HERE, "conv_ref.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add anywhere in the reference sums.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(source: str = SOURCE, output: str = LIBRARY, conv_source: str = CONV_SOURCE) -> str:
    """Compile the reference with gcc; returns the path of the shared object."""
    tmp = output + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, conv_source, "-lm"], check=True)
    os.replace(tmp, output)
    return output


_lib = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load (building first if absent) the reference shared object."""
    global _lib
    if path == LIBRARY and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(output=path)
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int)
    lib.oracle_sgemm.restype = ctypes.c_int
    lib.oracle_sgemm.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        f32p, ctypes.c_int, f32p, ctypes.c_int, ctypes.c_float,
        f32p, ctypes.c_int, f64p, ctypes.c_int,
    ]
    lib.oracle_sgemm_points.restype = None
    lib.oracle_sgemm_points.argtypes = [
        ctypes.c_int, ctypes.c_float, f32p, ctypes.c_int, f32p, ctypes.c_int,
        ctypes.c_float, f32p, ctypes.c_int, ctypes.c_int, i32p, i32p, f32p, f64p,
    ]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    c_int, c_long = ctypes.c_int, ctypes.c_long
    lib.oracle_conv_out_size.restype = c_int
    lib.oracle_conv_out_size.argtypes = [c_int] * 4
    lib.oracle_im2col.restype = None
    lib.oracle_im2col.argtypes = [c_int] * 10 + [f32p, f32p, c_long]
    lib.oracle_conv2d.restype = c_int
    lib.oracle_conv2d.argtypes = ([c_int] * 11 + [ctypes.c_float, f32p, f32p, c_long,
                                                  ctypes.c_float, f32p, c_long, f64p, c_long])
    if path == LIBRARY:
        _lib = lib
    return lib


def _ld(x: np.ndarray, name: str) -> int:
    """Leading dimension of a row-major 2-D float32 view (rows may be padded)."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("%s must be a 2-D float32 array" % name)
    if x.size == 0:
        return max(1, x.shape[1])
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError("%s must have unit column stride" % name)
    if x.shape[0] > 1:
        if x.strides[0] % 4 != 0 or x.strides[0] < 4 * x.shape[1]:
            raise ValueError("%s has an unusable row stride" % name)
        return x.strides[0] // 4
    return max(1, x.shape[1])


def _fptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def sgemm(A: np.ndarray, B: np.ndarray, C: Optional[np.ndarray] = None,
          alpha: float = 1.0, beta: float = 0.0, with_absdot: bool = True,
          lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Return (out, absdot) with out = fl32(alpha*A@B + beta*C) elementwise.

    ``A`` (M x K), ``B`` (K x N) and ``C`` (M x N) are float32 arrays whose
    rows may be strided views into larger buffers.  ``C`` is copied, never
    modified; ``out`` is a view with C's leading dimension into a buffer
    whose padding columns hold NaN (and must still hold NaN afterwards).
    ``absdot[i, j] = sum_k |A[i,k] * B[k,j]|`` in float64.
    """
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    if C is None:
        out = np.zeros((M, N), dtype=np.float32)
        ldc = max(1, N)
    else:
        if C.shape != (M, N):
            raise ValueError("C has the wrong shape")
        # Keep C's row pitch: the copy is made into a buffer of the same
        # leading dimension whose padding holds NaN, so the reference is run
        # with that ldc and must leave the padding alone.
        ldc = _ld(C, "C")
        buf = np.full((M, ldc), np.nan, dtype=np.float32)
        buf[:, :N] = C
        out = buf[:, :N]
    t = np.zeros((M, N), dtype=np.float64) if with_absdot else None
    if M == 0 or N == 0:
        return out, t
    # Empty K: hand the C code a valid dummy pointer; it reads nothing.
    dummy = np.zeros(1, dtype=np.float32)
    a = A if A.size else dummy.reshape(1, 1)
    b = B if B.size else dummy.reshape(1, 1)
    rc = lib.oracle_sgemm(
        M, N, K, ctypes.c_float(alpha), _fptr(a), lda, _fptr(b), ldb,
        ctypes.c_float(beta), _fptr(out), ldc,
        t.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if t is not None else None,
        N)
    if rc != 0:
        raise MemoryError("reference SGEMM could not allocate its row buffers")
    return out, t


def sgemm_points(A: np.ndarray, B: np.ndarray, C: Optional[np.ndarray],
                 alpha: float, beta: float, rows: np.ndarray, cols: np.ndarray,
                 lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Reference values at the given (row, col) pairs only.

    Returns (out, absdot), each of length len(rows).  ``C`` holds the values
    before the call and is read only when beta != 0.
    """
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample point outside the M x N output")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    out = np.empty(rows.size, dtype=np.float32)
    t = np.empty(rows.size, dtype=np.float64)
    if beta != 0.0:
        if C is None or C.shape != (M, N):
            raise ValueError("beta != 0 needs C of shape (M, N)")
        cptr, ldc = _fptr(C), _ld(C, "C")
    else:
        cptr, ldc = None, max(1, N)
    dummy = np.zeros(1, dtype=np.float32)
    a = A if A.size else dummy.reshape(1, 1)
    b = B if B.size else dummy.reshape(1, 1)
    i32p = ctypes.POINTER(ctypes.c_int)
    lib.oracle_sgemm_points(
        K, ctypes.c_float(alpha), _fptr(a), lda, _fptr(b), ldb, ctypes.c_float(beta),
        cptr, ldc, rows.size, rows.ctypes.data_as(i32p), cols.ctypes.data_as(i32p),
        _fptr(out), t.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out, t


def num_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    """Threads the reference's OpenMP runtime uses."""
    return int((lib or load()).oracle_num_threads())


def tolerance(alpha: float, beta: float, absdot: np.ndarray, c_before) -> np.ndarray:
    """Per-element bound |gpu - ref| <= 1e-5 * (|alpha| * sum|a*b| + |beta * c|) + 1e-6.

    This is the library's accuracy contract with the alpha and beta terms
    folded in; at alpha = 1, beta = 0 it is 1e-5 * sum_k |a_ik * b_kj| + 1e-6.
    """
    scale = abs(float(alpha)) * np.asarray(absdot, dtype=np.float64)
    if beta != 0.0:
        scale = scale + np.abs(float(beta) * np.asarray(c_before, dtype=np.float64))
    return 1e-5 * scale + 1e-6


def conv_out_size(size: int, k: int, stride: int, pad: int,
                  lib: Optional[ctypes.CDLL] = None) -> int:
    """Output extent along one axis: (size + 2 pad - k) // stride + 1."""
    if size + 2 * pad < k or stride < 1 or k < 1:
        raise ValueError("filter larger than the padded input, or bad stride")
    return int((lib or load()).oracle_conv_out_size(size, k, stride, pad))


def _geometry(X, R, S, stride, pad, lib=None):
    if X.dtype != np.float32 or X.ndim != 4 or not X.flags.c_contiguous:
        raise TypeError("X must be a packed (batch, C, H, W) float32 array")
    sh, sw = (stride, stride) if np.isscalar(stride) else stride
    ph, pw = (pad, pad) if np.isscalar(pad) else pad
    batch, C, H, W = X.shape
    OH, OW = conv_out_size(H, R, sh, ph, lib), conv_out_size(W, S, sw, pw, lib)
    return batch, C, H, W, int(sh), int(sw), int(ph), int(pw), OH, OW


def im2col(X: np.ndarray, R: int, S: int, stride=1, pad=0,
           lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """The (C*R*S) x (batch*OH*OW) matrix of taps of the convolution of X
    (packed NCHW float32) with an R x S filter: row k = (c*R + r)*S + s,
    column n = (b*OH + oh)*OW + ow; zeros where a tap leaves the image."""
    lib = lib or load()
    batch, C, H, W, sh, sw, ph, pw, OH, OW = _geometry(X, R, S, stride, pad, lib)
    B = np.empty((C * R * S, batch * OH * OW), dtype=np.float32)
    if B.size:
        lib.oracle_im2col(batch, C, H, W, R, S, sh, sw, ph, pw, _fptr(X), _fptr(B), B.shape[1])
    return B


def conv2d(X: np.ndarray, Wt: np.ndarray, R: int, S: int, stride=1, pad=0,
           Y: Optional[np.ndarray] = None, alpha: float = 1.0, beta: float = 0.0,
           with_absdot: bool = True,
           lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Return (out, absdot): out = fl32(alpha * conv(X, F) + beta * Y) with
    X packed (batch, C, H, W), the filters as the M x (C*R*S) matrix Wt (rows
    may be strided, F[m][c][r][s] at Wt[m, (c*R + r)*S + s]) and out an
    M x (batch*OH*OW) matrix in (b, oh, ow) column order, as the lowered
    product writes it.  Y (same shape, read only when beta != 0) is copied,
    never modified.  absdot[m, n] = sum_k |w * x| in float64."""
    lib = lib or load()
    batch, C, H, W, sh, sw, ph, pw, OH, OW = _geometry(X, R, S, stride, pad, lib)
    M, K = Wt.shape
    if K != C * R * S:
        raise ValueError("Wt must have C*R*S columns")
    ldw = _ld(Wt, "Wt")
    N = batch * OH * OW
    out = np.zeros((M, N), dtype=np.float32) if Y is None else np.array(Y, dtype=np.float32)
    if out.shape != (M, N):
        raise ValueError("Y has the wrong shape")
    t = np.zeros((M, N), dtype=np.float64) if with_absdot else None
    if M == 0 or N == 0:
        return out, t
    rc = lib.oracle_conv2d(batch, C, H, W, M, R, S, sh, sw, ph, pw, ctypes.c_float(alpha),
                           _fptr(X), _fptr(Wt), ldw, ctypes.c_float(beta), _fptr(out), N,
                           t.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
                           if t is not None else None, N)
    if rc != 0:
        raise MemoryError("reference convolution could not allocate its row buffers")
    return out, t
