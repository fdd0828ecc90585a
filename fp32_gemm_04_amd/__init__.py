"""Python binding of libsgemm, the MI355X single-precision GEMM.

Argument marshalling only: every step of the product runs in the HIP
kernels of ``libsgemm.so`` (built from ``csrc/`` by ``_build.py``).  If the
library is missing, importing this package raises; there is no fallback.

The functions have the names and arguments of the C ABI in
``include/sgemm.h``; ``gemm`` is a convenience that takes torch tensors and
passes their data pointers, leading dimensions and the current stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libsgemm.so")

SGEMM_VARIANT_AUTO = 0
SGEMM_VARIANT_MFMA = 1
SGEMM_VARIANT_VALU = 2
SGEMM_VARIANT_SKINNY = 3
SGEMM_VARIANT_MFMA_TILE = 16
SGEMM_VARIANT_LADDER = 32
SGEMM_VARIANT_STREAMK_TILE = 48
SGEMM_LADDER_RUNGS = 8
LADDER_RUNG_NAMES = ("naive", "coalesced", "lds", "tile1d", "tile2d", "regcache", "vec4", "dbuf")
SGEMM_ERR_BAD_VARIANT = -100
SGEMM_ERR_VARIANT_SHAPE = -101
SGEMM_ERR_WORKSPACE = -102
SGEMM_ERR_NO_SLOT = -103
SGEMM_ERR_CAPTURING = -104

SCONV_VARIANT_AUTO = 0
SCONV_VARIANT_STEM = 1
SCONV_VARIANT_GENERAL = 2
SCONV_VARIANT_TILE = 3
SCONV_VARIANT_DIRECT = 4
SCONV_VARIANT_TAP = 5

EXPORTS = ("sgemm_f32", "sgemm_f32_variant", "sgemm_plan", "sgemm_tune", "sgemm_tune_reset",
           "sgemm_num_mfma_tiles", "sgemm_status_string",
           # include/sconv.h
           "sconv2d_f32", "sconv2d_f32_variant", "sgemm_im2col_f32", "sconv2d_plan",
           "sconv2d_num_stem_kernels")

if not os.path.exists(LIBRARY):
    raise ImportError("libsgemm.so is not built; run __graft_entry__.build() "
                      "(or python fp32_gemm_04_amd/_build.py)")

# torch must be loaded first.  Its wheel carries its own HIP runtime
# (libamdhip64, soname libamdhip64.so.7, found through torch's RPATH as
# "libamdhip64.so"); libsgemm asks for "libamdhip64.so.7", which then
# resolves to that same already-loaded runtime.  Loaded the other way round,
# the process would hold two HIP runtimes, and torch's streams and memory
# would be foreign to the one libsgemm calls.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIBRARY)

_gemm_args = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
              ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
              ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
_lib.sgemm_f32.restype = ctypes.c_int
_lib.sgemm_f32.argtypes = _gemm_args
_lib.sgemm_f32_variant.restype = ctypes.c_int
_lib.sgemm_f32_variant.argtypes = [ctypes.c_int] + _gemm_args
_lib.sgemm_plan.restype = ctypes.c_int
_lib.sgemm_plan.argtypes = [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                                                 ctypes.c_char_p, ctypes.c_int]
_lib.sgemm_tune.restype = ctypes.c_int
_lib.sgemm_tune.argtypes = _gemm_args + [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_float)]
_lib.sgemm_tune_reset.restype = None
_lib.sgemm_tune_reset.argtypes = []
_lib.sgemm_num_mfma_tiles.restype = ctypes.c_int
_lib.sgemm_num_mfma_tiles.argtypes = []
_lib.sgemm_status_string.restype = ctypes.c_char_p
_lib.sgemm_status_string.argtypes = [ctypes.c_int]
_conv_args = ([ctypes.c_int] * 11 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p])
_lib.sconv2d_f32.restype = ctypes.c_int
_lib.sconv2d_f32.argtypes = _conv_args
_lib.sconv2d_f32_variant.restype = ctypes.c_int
_lib.sconv2d_f32_variant.argtypes = [ctypes.c_int] + _conv_args
_lib.sgemm_im2col_f32.restype = ctypes.c_int
_lib.sgemm_im2col_f32.argtypes = ([ctypes.c_int] * 10 + [ctypes.c_void_p, ctypes.c_void_p,
                                                         ctypes.c_int, ctypes.c_void_p])
_lib.sconv2d_plan.restype = ctypes.c_int
_lib.sconv2d_plan.argtypes = [ctypes.c_int] * 13 + [ctypes.c_char_p, ctypes.c_int]
_lib.sconv2d_num_stem_kernels.restype = ctypes.c_int
_lib.sconv2d_num_stem_kernels.argtypes = []


class SgemmError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("sgemm failed with status %d: %s" % (status, sgemm_status_string(status)))
        self.status = status


def sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C ABI ``sgemm_f32``; pointers and stream are integers.  Returns the status."""
    return _lib.sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C ABI ``sgemm_f32_variant``.  Returns the status."""
    return _lib.sgemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_plan(variant, M, N, K, lda, ldb, ldc, alpha, num_cus):
    """C ABI ``sgemm_plan``.  Returns (status, text)."""
    buf = ctypes.create_string_buffer(256)
    rc = _lib.sgemm_plan(variant, M, N, K, lda, ldb, ldc, alpha, num_cus, buf, len(buf))
    return rc, buf.value.decode()


def sgemm_tune(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, reps=5):
    """C ABI ``sgemm_tune``.  Returns (status, chosen variant, microseconds per launch)."""
    chosen = ctypes.c_int(0)
    us = ctypes.c_float(0.0)
    rc = _lib.sgemm_tune(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, reps,
                         ctypes.byref(chosen), ctypes.byref(us))
    return rc, chosen.value, us.value


def sgemm_tune_reset() -> None:
    """C ABI ``sgemm_tune_reset``."""
    _lib.sgemm_tune_reset()


def sgemm_num_mfma_tiles() -> int:
    """C ABI ``sgemm_num_mfma_tiles``."""
    return _lib.sgemm_num_mfma_tiles()


def sgemm_status_string(status: int) -> str:
    return _lib.sgemm_status_string(status).decode()


def tune(A, B, C, alpha: float = 1.0, beta: float = 0.0, reps: int = 5, stream=None):
    """Tune the kernel choice for this problem (``sgemm_tune``) and compute
    C <- alpha*A@B + beta*C in place with the winner.  Returns (variant,
    microseconds per launch); raises SgemmError on a non-zero status."""
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    s = stream if stream is not None else torch.cuda.current_stream(C.device)
    rc, chosen, us = sgemm_tune(M, N, K, alpha, A.data_ptr(), _ld(A, "A"), B.data_ptr(),
                                _ld(B, "B"), beta, C.data_ptr(), _ld(C, "C"), s.cuda_stream, reps)
    if rc != 0:
        raise SgemmError(rc)
    return chosen, us


def _ld(t, name):
    if t.dim() != 2 or t.dtype.__repr__() != "torch.float32":
        raise TypeError("%s must be a 2-D float32 tensor" % name)
    if t.numel() and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit column stride" % name)
    if t.shape[0] > 1 and t.numel():
        return t.stride(0)
    return max(1, t.shape[1])


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant: int = SGEMM_VARIANT_AUTO,
         stream=None):
    """C <- alpha*A@B + beta*C in place, for float32 CUDA/HIP tensors.

    Rows may be padded (stride(0) >= columns).  Queues on ``stream`` (a
    torch stream) or the current stream; raises SgemmError on a non-zero
    status.
    """
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    s = stream if stream is not None else torch.cuda.current_stream(C.device)
    rc = _lib.sgemm_f32_variant(variant, M, N, K, alpha, A.data_ptr(), _ld(A, "A"),
                                B.data_ptr(), _ld(B, "B"), beta, C.data_ptr(), _ld(C, "C"),
                                s.cuda_stream)
    if rc != 0:
        raise SgemmError(rc)
    return C


# ------------------------------------------------------------ convolution

def sconv2d_f32(batch, channels, height, width, out_channels, kernel_h, kernel_w, stride_h,
                stride_w, pad_h, pad_w, alpha, X, Wt, ldw, beta, Y, ldy, stream=0) -> int:
    """C ABI ``sconv2d_f32``; pointers and stream are integers.  Returns the status."""
    return _lib.sconv2d_f32(batch, channels, height, width, out_channels, kernel_h, kernel_w,
                            stride_h, stride_w, pad_h, pad_w, alpha, X, Wt, ldw, beta, Y, ldy,
                            stream)


def sconv2d_f32_variant(variant, batch, channels, height, width, out_channels, kernel_h,
                        kernel_w, stride_h, stride_w, pad_h, pad_w, alpha, X, Wt, ldw, beta, Y,
                        ldy, stream=0) -> int:
    """C ABI ``sconv2d_f32_variant``.  Returns the status."""
    return _lib.sconv2d_f32_variant(variant, batch, channels, height, width, out_channels,
                                    kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, alpha,
                                    X, Wt, ldw, beta, Y, ldy, stream)


def sgemm_im2col_f32(batch, channels, height, width, kernel_h, kernel_w, stride_h, stride_w,
                     pad_h, pad_w, X, B, ldb, stream=0) -> int:
    """C ABI ``sgemm_im2col_f32``.  Returns the status."""
    return _lib.sgemm_im2col_f32(batch, channels, height, width, kernel_h, kernel_w, stride_h,
                                 stride_w, pad_h, pad_w, X, B, ldb, stream)


def sconv2d_plan(variant, batch, channels, height, width, out_channels, kernel_h, kernel_w,
                 stride_h, stride_w, pad_h, pad_w, num_cus):
    """C ABI ``sconv2d_plan``.  Returns (status, text)."""
    buf = ctypes.create_string_buffer(256)
    rc = _lib.sconv2d_plan(variant, batch, channels, height, width, out_channels, kernel_h,
                           kernel_w, stride_h, stride_w, pad_h, pad_w, num_cus, buf, len(buf))
    return rc, buf.value.decode()


def sconv2d_num_stem_kernels() -> int:
    """C ABI ``sconv2d_num_stem_kernels``."""
    return _lib.sconv2d_num_stem_kernels()


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def conv2d(X, Wt, kernel, stride=1, pad=0, Y=None, alpha: float = 1.0, beta: float = 0.0,
           variant: int = SCONV_VARIANT_AUTO, stream=None):
    """Y <- alpha * conv(X, filters) + beta * Y for float32 device tensors:
    X packed (batch, C, H, W); Wt the filters as an out_channels x (C*R*S)
    matrix (or (out_channels, C, R, S), packed); Y an out_channels x
    (batch*OH*OW) matrix (allocated, zero, when None).  Returns Y; raises
    SgemmError on a non-zero status."""
    import torch
    R, S = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    batch, C, H, W = X.shape
    if not X.is_contiguous():
        raise ValueError("X must be packed NCHW")
    M = Wt.shape[0]
    W2 = Wt.reshape(M, -1) if Wt.dim() == 4 else Wt
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    if Y is None:
        Y = torch.zeros((M, batch * OH * OW), dtype=torch.float32, device=X.device)
    s = stream if stream is not None else torch.cuda.current_stream(X.device)
    rc = _lib.sconv2d_f32_variant(variant, batch, C, H, W, M, R, S, sh, sw, ph, pw, alpha,
                                  X.data_ptr(), W2.data_ptr(), _ld(W2, "Wt"), beta, Y.data_ptr(),
                                  _ld(Y, "Y"), s.cuda_stream)
    if rc != 0:
        raise SgemmError(rc)
    return Y


def im2col(X, kernel, stride=1, pad=0, B=None, stream=None):
    """The (C*R*S) x (batch*OH*OW) im2col matrix of a packed NCHW float32
    device tensor (into B, allocated when None).  Returns B."""
    import torch
    R, S = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    batch, C, H, W = X.shape
    if not X.is_contiguous():
        raise ValueError("X must be packed NCHW")
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    if B is None:
        B = torch.empty((C * R * S, batch * OH * OW), dtype=torch.float32, device=X.device)
    s = stream if stream is not None else torch.cuda.current_stream(X.device)
    rc = _lib.sgemm_im2col_f32(batch, C, H, W, R, S, sh, sw, ph, pw, X.data_ptr(), B.data_ptr(),
                               _ld(B, "B"), s.cuda_stream)
    if rc != 0:
        raise SgemmError(rc)
    return B
