"""GPU parity of the convolution entry points against the CPU reference.

sconv2d_f32 (stem, matrix-core tile and general kernels) and sgemm_im2col_f32
run through the C ABI on seeded inputs; every output element is compared with the reference
convolution: bit for bit on integer data (all partial sums are small
integers, so any summation order gives the same float), within
1e-5 * (|alpha| sum|w x| + |beta y|) + 1e-6 on uniform data.  Bytes of Y
outside its window and of the im2col matrix outside its rows keep their NaN
guards.  The full-size cases are the two stem readings of the skinny
convolution-as-GEMM shapes: 128 images of 3 x 224 x 224, 64 filters of 7 x 7
at stride 2 pad 3 (the (64, 1605632, 147) product) and 32 filters of 3 x 3
at stride 2 pad 1 (the (32, 1605632, 27) product).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import GUARD, assert_bits_equal, assert_within_tolerance, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


def _ints(shape, seed):
    return np.random.default_rng(seed).integers(-4, 5, size=shape).astype(np.float32)


def _uniform(shape, seed):
    v = np.random.default_rng(seed).random(shape, dtype=np.float32)
    return (2 * v - 1).astype(np.float32)


class Flat:
    """A host array copied into a device buffer between NaN guard bands, the
    rows of a 2-D array optionally padded to a leading dimension (NaN)."""

    def __init__(self, host, ld=None):
        host = np.ascontiguousarray(host, np.float32)
        if host.ndim == 2:
            rows, cols = host.shape
            self.ld = cols if ld is None else ld
            body = np.full((rows, self.ld), np.nan, np.float32)
            body[:, :cols] = host
            self.shape = (rows, cols)
        else:
            body = host
            self.ld = None
            self.shape = host.shape
        flat = body.reshape(-1)
        self.buf = torch.full((GUARD + flat.size + GUARD,), float("nan"), device="cuda")
        if flat.size:
            self.buf[GUARD:GUARD + flat.size].copy_(torch.from_numpy(flat))
        self.n = flat.size

    @property
    def ptr(self):
        return self.buf.data_ptr() + 4 * GUARD

    def window(self):
        flat = self.buf.cpu().numpy()
        body = flat[GUARD:GUARD + self.n]
        if self.ld is None:
            return body.reshape(self.shape)
        rows, cols = self.shape
        return body.reshape(rows, self.ld)[:, :cols].copy()

    def outside_is_nan(self):
        flat = self.buf.cpu().numpy()
        ok = np.all(np.isnan(flat[:GUARD])) and np.all(np.isnan(flat[GUARD + self.n:]))
        if self.ld is not None and self.shape[1] < self.ld:
            rows, cols = self.shape
            ok = ok and np.all(np.isnan(flat[GUARD:GUARD + self.n].reshape(rows, self.ld)[:, cols:]))
        return bool(ok)


def run_conv(X, Wt, M, R, S, stride, pad, alpha=1.0, beta=0.0, Y0=None, variant=0,
             ldw=None, ldy=None):
    import fp32_gemm_04_amd as sg
    batch, C, H, W = X.shape
    sh, sw = stride
    ph, pw = pad
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    N = batch * OH * OW
    dX = Flat(X)
    dW = Flat(Wt, ldw)
    Yin = Y0 if Y0 is not None else np.full((M, N), np.nan, np.float32)
    dY = Flat(Yin, ldy)
    s = torch.cuda.current_stream()
    say("sconv2d variant=%d batch=%d C=%d H=%d W=%d M=%d R=%d S=%d stride=%s pad=%s alpha=%g beta=%g"
        % (variant, batch, C, H, W, M, R, S, stride, pad, alpha, beta))
    rc = sg.sconv2d_f32_variant(variant, batch, C, H, W, M, R, S, sh, sw, ph, pw, alpha, dX.ptr,
                                dW.ptr, dW.ld, beta, dY.ptr, dY.ld, s.cuda_stream)
    assert rc == 0, "status %d: %s" % (rc, sg.sgemm_status_string(rc))
    s.synchronize()
    assert dY.outside_is_nan(), "Y written outside its window"
    return dY.window()


def check(X, Wt, R, S, stride, pad, variant, exact, alpha=1.0, beta=0.0, Y0=None, **kw):
    M = Wt.shape[0]
    out = run_conv(X, Wt, M, R, S, stride, pad, alpha, beta, Y0, variant, **kw)
    ref, t = oracle.conv2d(X, Wt, R, S, stride, pad, Y=Y0, alpha=alpha, beta=beta,
                           with_absdot=not exact)
    if exact:
        assert_bits_equal(out, ref, "conv variant %d" % variant)
    else:
        assert_within_tolerance(out, ref, t, alpha, beta, Y0, "conv variant %d" % variant)
    return out


# (batch, C, H, W, M, R, S, stride, pad): assorted geometries for the general
# kernel, and stem geometries (3 channels, 7x7 / 3x3 at stride 2, outputs 85
# to 113 positions wide) with ragged strips, partial row blocks, widths that
# are not multiples of 4 and asymmetric padding.
GENERAL = [
    (1, 1, 5, 6, 1, 3, 3, (1, 1), (1, 1)),
    (2, 3, 9, 11, 4, 3, 3, (2, 2), (1, 1)),
    (1, 2, 10, 7, 3, 2, 4, (1, 2), (0, 1)),
    (3, 2, 7, 13, 70, 5, 3, (2, 1), (2, 0)),
    (1, 4, 8, 9, 65, 1, 1, (3, 2), (0, 0)),
    (2, 16, 17, 19, 33, 3, 3, (1, 1), (1, 1)),
    (1, 5, 12, 12, 130, 3, 5, (3, 3), (4, 6)),
]
STEM = [
    (2, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3)),
    (3, 3, 200, 190, 50, 7, 7, (2, 2), (3, 3)),
    (2, 3, 224, 224, 20, 7, 7, (2, 2), (3, 3)),
    (1, 3, 61, 222, 64, 7, 7, (2, 2), (2, 1)),
    (2, 3, 224, 224, 32, 3, 3, (2, 2), (1, 1)),
    (2, 3, 224, 224, 17, 3, 3, (2, 2), (1, 1)),
    (3, 3, 45, 181, 64, 3, 3, (2, 2), (0, 1)),
    (1, 3, 224, 227, 33, 3, 3, (2, 2), (1, 1)),
]

# Geometries for the matrix-core tile kernels: several tiles in both
# directions with ragged edges, channel counts that are not multiples of 16
# (5, 1, 20, 33), strides and paddings, batch > 1, 1x1 and 5x3 filters; the
# last is a 3x3 stride-1 layer with 128 channels at a size that still runs
# quickly on the reference.
TILE = [
    (2, 32, 30, 31, 200, 3, 3, (1, 1), (1, 1)),
    (1, 5, 40, 37, 130, 3, 3, (1, 1), (1, 1)),
    (3, 1, 33, 29, 64, 3, 3, (1, 1), (0, 0)),
    (1, 64, 57, 57, 129, 3, 3, (2, 2), (1, 1)),
    (2, 20, 23, 25, 70, 3, 3, (2, 1), (2, 0)),
    (2, 48, 20, 21, 96, 1, 1, (1, 1), (0, 0)),
    (1, 33, 15, 15, 260, 1, 1, (2, 2), (1, 1)),
    (2, 17, 21, 18, 40, 5, 3, (1, 2), (2, 1)),
    (1, 128, 36, 36, 384, 3, 3, (1, 1), (1, 1)),
]


def _plan(variant, g):
    import fp32_gemm_04_amd as sg
    batch, C, H, W, M, R, S, (sh, sw), (ph, pw) = g
    return sg.sconv2d_plan(variant, batch, C, H, W, M, R, S, sh, sw, ph, pw, 256)


def _direct_applies(g):
    return _plan(4, g)[0] == 0


def _tap_applies(g):
    return _plan(5, g)[0] == 0


def _applies(variant, g):
    return {4: _direct_applies, 5: _tap_applies}.get(variant, lambda g: True)(g)


def _stem_applies(g):
    import fp32_gemm_04_amd as sg
    batch, C, H, W, M, R, S, (sh, sw), (ph, pw) = g
    rc, plan = sg.sconv2d_plan(0, batch, C, H, W, M, R, S, sh, sw, ph, pw, 256)
    assert rc == 0
    return plan.startswith("stem")


@pytest.mark.parametrize("integer", [True, False], ids=["integer", "uniform"])
@pytest.mark.parametrize("variant", [0, 2, 3, 4, 5],
                         ids=["auto", "general", "tile", "direct", "tap"])
@pytest.mark.parametrize("g", GENERAL + STEM + TILE,
                         ids=[str(i) for i in range(len(GENERAL + STEM + TILE))])
def test_conv_small(g, variant, integer):
    if not _applies(variant, g):
        pytest.skip("form %d does not take this geometry" % variant)
    batch, C, H, W, M, R, S, stride, pad = g
    gen = _ints if integer else _uniform
    X = gen((batch, C, H, W), 11 + H)
    Wt = gen((M, C * R * S), 13 + W)
    check(X, Wt, R, S, stride, pad, variant, integer)


@pytest.mark.parametrize("g", STEM, ids=[str(i) for i in range(len(STEM))])
def test_stem_geometries_take_the_stem_kernel(g):
    import fp32_gemm_04_amd as sg
    assert _stem_applies(g), g
    batch, C, H, W, M, R, S, stride, pad = g
    X = _ints((batch, C, H, W), 21 + H)
    Wt = _ints((M, C * R * S), 23 + W)
    check(X, Wt, R, S, stride, pad, sg.SCONV_VARIANT_STEM, True, alpha=1.5, beta=0.5,
          Y0=_ints((M, batch * ((H + 2 * pad[0] - R) // stride[0] + 1)
                    * ((W + 2 * pad[1] - S) // stride[1] + 1)), 25))


@pytest.mark.parametrize("variant", [0, 2, 3, 4, 5],
                         ids=["auto", "general", "tile", "direct", "tap"])
def test_padded_leading_dimensions_and_beta(variant):
    for g in [STEM[1], GENERAL[3], STEM[6], TILE[0], TILE[3], TILE[5], TILE[6]]:
        if not _applies(variant, g):
            continue
        batch, C, H, W, M, R, S, stride, pad = g
        OH = (H + 2 * pad[0] - R) // stride[0] + 1
        OW = (W + 2 * pad[1] - S) // stride[1] + 1
        X = _ints((batch, C, H, W), 31)
        Wt = _ints((M, C * R * S), 32)
        Y0 = _ints((M, batch * OH * OW), 33)
        # The direct forms need filter rows 16-byte aligned: pad by 4 there.
        check(X, Wt, R, S, stride, pad, variant, True, alpha=-1.0, beta=2.0, Y0=Y0,
              ldw=C * R * S + (4 if variant in (4, 5) else 3), ldy=batch * OH * OW + 5)


def test_direct_form_needs_aligned_filters():
    """The call takes the register-staged tile form when the filter rows are
    not 16-byte aligned, the direct form otherwise; both match the reference."""
    import fp32_gemm_04_amd as sg
    g = TILE[0]
    batch, C, H, W, M, R, S, (sh, sw), (ph, pw) = g
    K = C * R * S
    assert _direct_applies(g)
    X = _ints((batch, C, H, W), 35)
    Wt = _ints((M, K), 36)
    for ldw in (K + 1, K + 4):
        check(X, Wt, R, S, (sh, sw), (ph, pw), 0, True, ldw=ldw)
    s = torch.cuda.current_stream()
    rc = sg.sconv2d_f32_variant(4, batch, C, H, W, M, R, S, sh, sw, ph, pw, 1.0, 0x1000,
                                0x2004, K + 4, 0.0, 0x3000, batch * H * W, s.cuda_stream)
    assert rc == sg.SGEMM_ERR_VARIANT_SHAPE  # misaligned filters: refused before any launch


def test_beta_zero_does_not_read_y_and_alpha_zero_scales():
    batch, C, H, W, M, R, S, stride, pad = STEM[0]
    OH = (H + 2 * pad[0] - R) // stride[0] + 1
    OW = (W + 2 * pad[1] - S) // stride[1] + 1
    X = _ints((batch, C, H, W), 41)
    Wt = _ints((M, C * R * S), 42)
    for variant in (0, 2):
        out = check(X, Wt, R, S, stride, pad, variant, True)  # Y starts as NaN
        assert not np.isnan(out).any()
    g = TILE[1]
    Xt = _ints(g[:4], 44)
    Wtt = _ints((g[4], g[1] * 9), 45)
    out = check(Xt, Wtt, 3, 3, g[7], g[8], 3, True)
    assert not np.isnan(out).any()
    Y0 = _ints((M, batch * OH * OW), 43)
    out = run_conv(X, Wt, M, R, S, stride, pad, alpha=0.0, beta=-0.5, Y0=Y0)
    assert np.array_equal(out, -0.5 * Y0)


def test_im2col_matches_reference_and_feeds_sgemm():
    """sgemm_im2col_f32 writes the reference's im2col matrix bit for bit
    (128-bit path, and 32-bit with a padded, misaligned ldb); sgemm_f32 on it
    equals sconv2d_f32 on integer data."""
    import fp32_gemm_04_amd as sg
    s = torch.cuda.current_stream()
    for i, g in enumerate(GENERAL + STEM[:3]):
        batch, C, H, W, M, R, S, (sh, sw), (ph, pw) = g
        X = _uniform((batch, C, H, W), 50 + i)
        ref = oracle.im2col(X, R, S, (sh, sw), (ph, pw))
        K, N = ref.shape
        for ld in (N, N + 3):
            dX = Flat(X)
            dB = Flat(np.full((K, N), np.nan, np.float32), ld)
            say("im2col case %d ldb=%d" % (i, ld))
            rc = sg.sgemm_im2col_f32(batch, C, H, W, R, S, sh, sw, ph, pw, dX.ptr, dB.ptr, ld,
                                     s.cuda_stream)
            assert rc == 0, sg.sgemm_status_string(rc)
            s.synchronize()
            assert_bits_equal(dB.window(), ref, "im2col case %d" % i)
            assert dB.outside_is_nan()
        Xi = _ints((batch, C, H, W), 60 + i)
        Wi = _ints((M, K), 61 + i)
        Bi = torch.from_numpy(oracle.im2col(Xi, R, S, (sh, sw), (ph, pw))).cuda()
        dWi = torch.from_numpy(Wi).cuda()
        Yg = torch.empty((M, N), device="cuda")
        sg.gemm(dWi, Bi, Yg)
        conv = run_conv(Xi, Wi, M, R, S, (sh, sw), (ph, pw))
        assert_bits_equal(Yg.cpu().numpy(), conv, "im2col + sgemm against sconv2d, case %d" % i)


# The two stem readings at full size (N = 128 * 112 * 112 = 1605632), and
# the other readings through the kernel the call picks (the tap form; for
# the 1x1 reading the GEMM on the input in place), the 16-tap direct form,
# the register-staged tile kernel and the general kernel, all against one
# reference result.
@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
@pytest.mark.parametrize("case", workloads.CONV_STEMS + workloads.CONV_MID,
                         ids=[c.name for c in workloads.CONV_STEMS + workloads.CONV_MID])
def test_full_size_readings(case, integer):
    import fp32_gemm_04_amd as sg
    X, Wt = workloads.conv_operands(case, integer)
    g = case.geometry
    b, C, H, W, M, R, S, sh, sw, ph, pw = g
    stride, pad = (sh, sw), (ph, pw)
    rc, plan = sg.sconv2d_plan(0, b, C, H, W, M, R, S, sh, sw, ph, pw, 256)
    assert rc == 0
    if case in workloads.CONV_STEMS:
        assert plan.startswith("stem"), plan
        variants = [0]
    else:
        # 3x3 readings: the tap form; the 1x1 reading: one product on X in place
        assert plan.startswith("gemm" if case.R == 1 else "tap"), plan
        variants = [0, 4, 3, 2]
    ref, t = oracle.conv2d(X, Wt, R, S, stride, pad, with_absdot=not integer)
    for variant in variants:
        out = run_conv(X, Wt, M, R, S, stride, pad, variant=variant)
        what = "%s variant %d" % (case.name, variant)
        if integer:
            assert_bits_equal(out, ref, what)
        else:
            assert_within_tolerance(out, ref, t, 1.0, 0.0, None, what)
        assert out.shape == (case.M, case.N)
        say("%s %s: %d elements" % (what, "integer" if integer else "uniform", out.size))
