"""Pins of the CPU reference convolution and im2col to facts outside them.

Each pin is a plain function ``pin_xxx(lib)`` that raises AssertionError when
the reference loaded as ``lib`` disagrees with an independent computation:
scipy's 2-D correlation of each channel, numpy sliding windows over an
explicitly zero-padded input, a 1x1 convolution as a numpy matrix product,
and closed forms (all-ones data count the taps inside the image; a one-hot
filter shifts the input).  ``tests/test_oracle_conv.py`` runs them against
the real reference; ``tests/test_oracle_mutants.py`` runs them against copies
with a planted mistake.

Integer-valued data make every comparison exact: all partial sums are small
integers, so any summation order gives the same float.
"""
from __future__ import annotations

import numpy as np

import oracle

# (batch, C, H, W, M, R, S, (sh, sw), (ph, pw)): odd sizes, unequal strides
# and pads, filters wider than the pad, a stride larger than the filter, and
# the two stem geometries of the convolution-as-GEMM shapes at reduced size.
GEOMETRIES = [
    (1, 1, 5, 6, 1, 3, 3, (1, 1), (1, 1)),
    (2, 3, 9, 11, 4, 3, 3, (2, 2), (1, 1)),
    (1, 2, 10, 7, 3, 2, 4, (1, 2), (0, 1)),
    (2, 3, 16, 16, 5, 7, 7, (2, 2), (3, 3)),
    (1, 4, 8, 9, 2, 1, 1, (3, 2), (0, 0)),
    (3, 2, 7, 13, 3, 5, 3, (2, 1), (2, 0)),
    (1, 3, 12, 12, 2, 3, 5, (3, 3), (1, 2)),
]


def _ints(shape, seed):
    return np.random.default_rng(seed).integers(-4, 5, size=shape).astype(np.float32)


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def _windows_reference(X, F, stride, pad):
    """Convolution by explicit zero padding and sliding windows, in float64;
    returns the M x (batch*OH*OW) matrix in (b, oh, ow) column order."""
    (sh, sw), (ph, pw) = stride, pad
    R, S = F.shape[2], F.shape[3]
    Xp = np.pad(X.astype(np.float64), ((0, 0), (0, 0), (ph, ph), (pw, pw)))
    win = np.lib.stride_tricks.sliding_window_view(Xp, (R, S), axis=(2, 3))[:, :, ::sh, ::sw]
    out = np.einsum("bchwrs,mcrs->mbhw", win, F.astype(np.float64))
    return out.reshape(F.shape[0], -1)


def pin_conv_matches_scipy_correlation(lib):
    """Per output channel, the sum over input channels of scipy's 2-D
    correlation of the zero-padded channel with the filter, sampled at the
    stride: exact on integer data."""
    from scipy.signal import correlate2d
    for i, (batch, C, H, W, M, R, S, st, pd) in enumerate(GEOMETRIES):
        X = _ints((batch, C, H, W), 100 + i)
        F = _ints((M, C, R, S), 200 + i)
        out, _ = oracle.conv2d(X, F.reshape(M, -1), R, S, st, pd, lib=lib)
        (sh, sw), (ph, pw) = st, pd
        OH = (H + 2 * ph - R) // sh + 1
        OW = (W + 2 * pw - S) // sw + 1
        expect = np.zeros((M, batch, OH, OW))
        for m in range(M):
            for b in range(batch):
                for c in range(C):
                    xp = np.pad(X[b, c].astype(np.float64), ((ph, ph), (pw, pw)))
                    full = correlate2d(xp, F[m, c].astype(np.float64), mode="valid")
                    expect[m, b] += full[::sh, ::sw][:OH, :OW]
        assert out.shape == (M, batch * OH * OW), (i, out.shape)
        assert np.array_equal(out, expect.reshape(M, -1).astype(np.float32)), i


def pin_conv_matches_padded_windows(lib):
    """Uniform data: the reference equals the float64 sliding-window result
    rounded to float (both are the exact sum up to double rounding)."""
    for i, (batch, C, H, W, M, R, S, st, pd) in enumerate(GEOMETRIES):
        rng = np.random.default_rng(300 + i)
        X = (2 * rng.random((batch, C, H, W), dtype=np.float32) - 1).astype(np.float32)
        F = (2 * rng.random((M, C, R, S), dtype=np.float32) - 1).astype(np.float32)
        out, t = oracle.conv2d(X, F.reshape(M, -1), R, S, st, pd, lib=lib)
        ref = _windows_reference(X, F, st, pd)
        tref = _windows_reference(np.abs(X), np.abs(F), st, pd)
        err = np.abs(out.astype(np.float64) - ref)
        assert np.all(err <= 2.0 ** -24 * np.abs(ref) + 1e-30), (i, float(err.max()))
        assert np.allclose(t, tref, rtol=1e-12, atol=0), i


def pin_one_by_one_is_matrix_product(lib):
    """A 1x1 filter at stride 1 without padding is the product of the weight
    matrix with each image's C x (H*W) matrix."""
    batch, C, H, W, M = 3, 5, 4, 7, 6
    X = _ints((batch, C, H, W), 400)
    Wt = _ints((M, C), 401)
    out, _ = oracle.conv2d(X, Wt, 1, 1, 1, 0, lib=lib)
    expect = np.concatenate([Wt.astype(np.int64) @ X[b].reshape(C, -1).astype(np.int64)
                             for b in range(batch)], axis=1)
    assert np.array_equal(out, expect.astype(np.float32))


def pin_ones_count_taps_inside(lib):
    """All-ones input and filter: each output is C times the number of filter
    taps that land inside the image, counted per axis in closed form."""
    for batch, C, H, W, M, R, S, (sh, sw), (ph, pw) in GEOMETRIES:
        X = np.ones((batch, C, H, W), np.float32)
        out, t = oracle.conv2d(X, np.ones((M, C * R * S), np.float32), R, S, (sh, sw),
                               (ph, pw), lib=lib)
        OH = (H + 2 * ph - R) // sh + 1
        OW = (W + 2 * pw - S) // sw + 1
        rows = np.array([sum(0 <= oh * sh - ph + r < H for r in range(R)) for oh in range(OH)])
        cols = np.array([sum(0 <= ow * sw - pw + s < W for s in range(S)) for ow in range(OW)])
        per_image = C * np.outer(rows, cols).reshape(-1)
        expect = np.tile(np.tile(per_image, batch), (M, 1)).astype(np.float32)
        assert np.array_equal(out, expect)
        assert np.array_equal(t, expect.astype(np.float64))


def pin_one_hot_filter_shifts_input(lib):
    """A filter with a single 1 at (c0, r0, s0) copies channel c0 of the input,
    shifted by (r0 - ph, s0 - pw) and sampled at the stride, zeros outside."""
    batch, C, H, W, M, R, S, (sh, sw), (ph, pw) = 2, 3, 9, 10, 1, 3, 4, (2, 1), (1, 2)
    X = _ints((batch, C, H, W), 500)
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    for c0, r0, s0 in [(0, 0, 0), (2, 1, 3), (1, 2, 1)]:
        F = np.zeros((1, C, R, S), np.float32)
        F[0, c0, r0, s0] = 1.0
        out, _ = oracle.conv2d(X, F.reshape(1, -1), R, S, (sh, sw), (ph, pw), lib=lib)
        Xp = np.pad(X[:, c0], ((0, 0), (ph, ph), (pw, pw)))
        expect = Xp[:, r0:r0 + sh * (OH - 1) + 1:sh, s0:s0 + sw * (OW - 1) + 1:sw]
        assert np.array_equal(out.reshape(batch, OH, OW), expect), (c0, r0, s0)


def pin_im2col_is_the_window_matrix(lib):
    """im2col's rows are the (c, r, s) taps and its columns the (b, oh, ow)
    positions of the padded sliding windows, bit for bit (pure data
    movement), and the product with the weights is the convolution."""
    for i, (batch, C, H, W, M, R, S, st, pd) in enumerate(GEOMETRIES):
        rng = np.random.default_rng(600 + i)
        X = (2 * rng.random((batch, C, H, W), dtype=np.float32) - 1).astype(np.float32)
        B = oracle.im2col(X, R, S, st, pd, lib=lib)
        (sh, sw), (ph, pw) = st, pd
        Xp = np.pad(X, ((0, 0), (0, 0), (ph, ph), (pw, pw)))
        win = np.lib.stride_tricks.sliding_window_view(Xp, (R, S), axis=(2, 3))[:, :, ::sh, ::sw]
        expect = win.transpose(1, 4, 5, 0, 2, 3).reshape(C * R * S, -1)
        assert np.array_equal(_bits(B), _bits(expect)), i
        F = (2 * rng.random((M, C * R * S), dtype=np.float32) - 1).astype(np.float32)
        conv, _ = oracle.conv2d(X, F, R, S, st, pd, lib=lib)
        gemm, _ = oracle.sgemm(F, B, lib=lib)
        assert np.array_equal(_bits(conv), _bits(gemm)), i


def pin_conv_alpha_beta(lib):
    """Integer data: alpha = 1.5, beta = 0.5 gives 1.5 conv + 0.5 Y exactly;
    beta = 0 leaves NaN in Y unread; alpha = 0 gives beta * Y."""
    batch, C, H, W, M, R, S, st, pd = GEOMETRIES[1]
    X = _ints((batch, C, H, W), 700)
    F = _ints((M, C * R * S), 701)
    plain, _ = oracle.conv2d(X, F, R, S, st, pd, lib=lib)
    Y = _ints(plain.shape, 702)
    got, t = oracle.conv2d(X, F, R, S, st, pd, Y=Y, alpha=1.5, beta=0.5, lib=lib)
    assert np.array_equal(got, 1.5 * plain + 0.5 * Y)
    nan = np.full(plain.shape, np.nan, np.float32)
    got0, _ = oracle.conv2d(X, F, R, S, st, pd, Y=nan, alpha=1.0, beta=0.0, lib=lib)
    assert np.array_equal(got0, plain)
    gota, _ = oracle.conv2d(X, F, R, S, st, pd, Y=Y, alpha=0.0, beta=-2.0, lib=lib)
    assert np.array_equal(gota, -2.0 * Y)


def pin_zero_padding_multiplies(lib):
    """An infinite weight on tap (0, 0, 0) with a positive input: the product
    with the zeros of the padding is NaN exactly where that tap falls outside
    the image (top rows or left columns of the output), +inf elsewhere."""
    batch, C, H, W, R, S, (sh, sw), (ph, pw) = 1, 1, 6, 7, 3, 3, (1, 2), (1, 1)
    X = np.ones((batch, C, H, W), np.float32)
    F = np.zeros((1, R * S), np.float32)
    F[0, 0] = np.inf
    out, _ = oracle.conv2d(X, F, R, S, (sh, sw), (ph, pw), lib=lib)
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    o = out.reshape(OH, OW)
    outside = np.zeros((OH, OW), bool)
    outside[[oh for oh in range(OH) if oh * sh - ph < 0], :] = True
    outside[:, [ow for ow in range(OW) if ow * sw - pw < 0]] = True
    assert np.all(np.isnan(o[outside])) and np.all(o[~outside] == np.inf)


def pin_stem_output_sizes(lib):
    """The two stem readings give the 112 x 112 outputs the GEMM shapes imply
    (N = 128 * 112 * 112 = 1605632): 224 input, 7x7 stride 2 pad 3 and 3x3
    stride 2 pad 1."""
    assert oracle.conv_out_size(224, 7, 2, 3, lib) == 112
    assert oracle.conv_out_size(224, 3, 2, 1, lib) == 112
    assert 128 * 112 * 112 == 1605632
    for size, k, s, p in [(5, 3, 1, 1), (9, 3, 2, 1), (16, 7, 2, 3), (8, 1, 3, 0), (7, 5, 2, 2)]:
        assert oracle.conv_out_size(size, k, s, p, lib) == (size + 2 * p - k) // s + 1


ALL_PINS = [
    pin_conv_matches_scipy_correlation,
    pin_conv_matches_padded_windows,
    pin_one_by_one_is_matrix_product,
    pin_ones_count_taps_inside,
    pin_one_hot_filter_shifts_input,
    pin_im2col_is_the_window_matrix,
    pin_conv_alpha_beta,
    pin_zero_padding_multiplies,
    pin_stem_output_sizes,
]
