"""Seeded synthetic inputs for the SGEMM workloads.

This module only draws random numbers and names shapes; it holds none of the
GEMM arithmetic.  Both the GPU tests/benchmark and the CPU reference take
their inputs from here, so the two sides see identical bytes.

Shapes and value distributions:
  * square products from the NVIDIA_SGEMM_PRACTICE README (results table at
    size 5120) and the cnblogs "matmul_opt.cu" demo (1024 x 1024);
  * the six im2col convolution shapes of the UNIVERSAL_SGEMM_CUDA README
    ("Results" section), split into the three skinny-K ones and the three
    mid-size ones.  The page measures networks it does not name; uniform
    random values of the same shapes stand in for those activations, since
    GEMM run time does not depend on finite, normal values.
Values are iid uniform on [-1, 1) (``2*U[0,1) - 1``), or integers drawn
uniformly from {-4, ..., 4} for the bit-exact variant.

Seeds: ``10000*config + 100*sub + role`` with role 0 = A, 1 = B, 2 = C, plus
50 for the integer variant.

The convolution readings of those shapes (``ConvCase``; the page names no
layers, so these geometries are readings of the shapes' factors): 128
images of 3 x 224 x 224 with 64 filters of 7 x 7 at stride 2, pad 3, give
the (64, 1605632, 147) product, and with 32 filters of 3 x 3 at stride 2,
pad 1 the (32, 1605632, 27) one; one 128-channel image of 119 x 119 (or
208 x 208) with 384 (or 256) filters of 3 x 3 at stride 1, pad 1 gives the
(384, 14161, 1152) (or (256, 43264, 1152)) product.  Inputs and filters are
uniform on [-1, 1) (or integers in [-4, 4]); seeds as above with config 5,
role 0 = filters, 1 = input.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Case:
    """One GEMM problem: C (M x N) <- alpha * A (M x K) @ B (K x N) + beta * C."""
    config: int
    sub: int
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    c_preload: bool
    name: str

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> float:
        """Bytes the product must move at least once: A, B and C written,
        plus C read when beta != 0."""
        b = 4.0 * (self.M * self.K + self.K * self.N + self.M * self.N)
        if self.beta != 0.0:
            b += 4.0 * self.M * self.N
        return b


def _sweep() -> List[Case]:
    return [Case(2, i, n, n, n, 1.5, 0.5, True, "sweep%d" % n)
            for i, n in enumerate(range(256, 5121, 256))]


SMALL = Case(0, 0, 256, 256, 256, 1.0, 0.0, False, "square256")
SQUARE1024 = Case(1, 0, 1024, 1024, 1024, 1.0, 0.0, True, "square1024_cpreload")
SWEEP = _sweep()
HEADLINE = SWEEP[-1]                       # 5120^3, alpha 1.5, beta 0.5
SKINNY = [
    Case(3, 0, 32, 1605632, 27, 1.0, 0.0, False, "im2col_32x1605632x27"),
    Case(3, 1, 64, 1605632, 147, 1.0, 0.0, False, "im2col_64x1605632x147"),
    Case(3, 2, 64, 559104, 147, 1.0, 0.0, False, "im2col_64x559104x147"),
]
MID = [
    Case(4, 0, 384, 14161, 1152, 1.0, 0.0, False, "im2col_384x14161x1152"),
    Case(4, 1, 256, 43264, 1152, 1.0, 0.0, False, "im2col_256x43264x1152"),
    Case(4, 2, 256, 50176, 1024, 1.0, 0.0, False, "im2col_256x50176x1024"),
]
ALL: List[Case] = [SMALL, SQUARE1024] + SWEEP + SKINNY + MID


def seed(case: Case, role: int, integer: bool = False) -> int:
    """Seed for operand ``role`` (0 = A, 1 = B, 2 = C) of ``case``."""
    return 10000 * case.config + 100 * case.sub + role + (50 if integer else 0)


def uniform(rows: int, cols: int, seed_value: int, ld: Optional[int] = None,
            fill: float = 0.0) -> np.ndarray:
    """rows x cols float32 values, iid uniform on [-1, 1).

    With ``ld`` > cols, the result is a view into a rows x ld buffer whose
    padding columns hold ``fill``.
    """
    rng = np.random.default_rng(seed_value)
    vals = rng.random((rows, cols), dtype=np.float32)
    vals *= np.float32(2.0)
    vals -= np.float32(1.0)
    return _embed(vals, ld, fill)


def integers(rows: int, cols: int, seed_value: int, ld: Optional[int] = None,
             fill: float = 0.0, low: int = -4, high: int = 4) -> np.ndarray:
    """rows x cols float32 values, integers drawn uniformly from [low, high]."""
    rng = np.random.default_rng(seed_value)
    vals = rng.integers(low, high + 1, size=(rows, cols), dtype=np.int32).astype(np.float32)
    return _embed(vals, ld, fill)


def _embed(vals: np.ndarray, ld: Optional[int], fill: float) -> np.ndarray:
    rows, cols = vals.shape
    if ld is None or ld == cols:
        return vals
    if ld < cols:
        raise ValueError("ld smaller than the number of columns")
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = vals
    return buf[:, :cols]


def operands(case: Case, integer: bool = False) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """(A, B, C-before) for a case; C is None when the case does not preload C."""
    gen = integers if integer else uniform
    A = gen(case.M, case.K, seed(case, 0, integer))
    B = gen(case.K, case.N, seed(case, 1, integer))
    C = gen(case.M, case.N, seed(case, 2, integer)) if case.c_preload else None
    return A, B, C


def device_integers(rows: int, cols: int, seed_value: int):
    """rows x cols float32 integers in [-4, 4] drawn on the GPU (torch's seeded
    generator), for operands too large to draw on the host; the tests copy
    the rows or columns they check back to the host for the reference."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed_value)
    return torch.randint(-4, 5, (rows, cols), generator=gen, device="cuda",
                         dtype=torch.float32)


@dataclass(frozen=True)
class ConvCase:
    """A convolution: `batch` images of C x H x W, M filters of C x R x S,
    strides (sh, sw), zero padding (ph, pw); the output is the M x N matrix
    (N = batch*OH*OW) of the lowered product with K = C*R*S."""
    sub: int
    name: str
    batch: int
    C: int
    H: int
    W: int
    M: int
    R: int
    S: int
    sh: int
    sw: int
    ph: int
    pw: int

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.ph - self.R) // self.sh + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pw - self.S) // self.sw + 1

    @property
    def N(self) -> int:
        return self.batch * self.OH * self.OW

    @property
    def K(self) -> int:
        return self.C * self.R * self.S

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> float:
        """Input, filters and output, each moved once (beta = 0)."""
        return 4.0 * (self.batch * self.C * self.H * self.W + self.M * self.K + self.M * self.N)

    @property
    def geometry(self) -> Tuple[int, ...]:
        return (self.batch, self.C, self.H, self.W, self.M, self.R, self.S, self.sh, self.sw,
                self.ph, self.pw)


CONV_STEMS = [
    ConvCase(0, "conv7x7s2_64x1605632x147", 128, 3, 224, 224, 64, 7, 7, 2, 2, 3, 3),
    ConvCase(1, "conv3x3s2_32x1605632x27", 128, 3, 224, 224, 32, 3, 3, 2, 2, 1, 1),
]
CONV_MID = [
    ConvCase(2, "conv3x3s1_384x14161x1152", 1, 128, 119, 119, 384, 3, 3, 1, 1, 1, 1),
    ConvCase(3, "conv3x3s1_256x43264x1152", 1, 128, 208, 208, 256, 3, 3, 1, 1, 1, 1),
    # (256, 50176, 1024): one 224 x 224 output (50176 = 224^2) of a 1 x 1 filter over 1024
    # channels, the plainest geometry with those factors
    ConvCase(4, "conv1x1_256x50176x1024", 1, 1024, 224, 224, 256, 1, 1, 1, 1, 0, 0),
]


def conv_operands(case: ConvCase, integer: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(X packed NCHW, filters as the M x K matrix) for a convolution case."""
    gen = integers if integer else uniform
    base = 10000 * 5 + 100 * case.sub + (50 if integer else 0)
    Wt = gen(case.M, case.K, base + 0)
    X = gen(case.batch * case.C, case.H * case.W, base + 1).reshape(case.batch, case.C, case.H,
                                                                      case.W)
    return np.ascontiguousarray(X), Wt
