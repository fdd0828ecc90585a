"""Seeded random convolutions through every implicit form that takes them.

Geometries (batch, channels, image size, output channels, filter size,
strides, padding) are drawn with one fixed seed, so every run draws the same
cases; each runs through the call's own choice and through every forced form
whose plan accepts it (general, register-staged tile, direct-to-LDS, tap),
with padded leading dimensions and alpha/beta drawn too.  Integer data: every
output element must equal the reference convolution bit for bit, and nothing
outside Y's window may change."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = (0, 2, 3, 4, 5)  # auto, general, tile, direct, tap


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


def _cases(count=96, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        R = int(rng.choice([1, 1, 3, 3, 3, 2, 5]))
        S = R if rng.random() < 0.8 else int(rng.choice([1, 3, 5]))
        sh, sw = (int(rng.integers(1, 3)), int(rng.integers(1, 3))) if rng.random() < 0.4 else (1, 1)
        ph, pw = int(rng.integers(0, R // 2 + 2)), int(rng.integers(0, S // 2 + 2))
        H = int(rng.integers(max(1, R - 2 * ph), 34))
        W = int(rng.integers(max(1, S - 2 * pw), 34))
        C = int(rng.choice([1, 3, 4, 8, 12, 16, 20, 32, 36, 48]))
        M = int(rng.integers(1, 260))
        batch = int(rng.integers(1, 4))
        if i % 8 == 7:  # large enough that the call itself picks a tile form
            H, W = int(rng.integers(40, 72)), int(rng.integers(40, 72))
            C, M, batch = int(rng.choice([16, 32, 64])), int(rng.integers(100, 400)), 2
        ldw_pad = int(rng.choice([0, 0, 4, 3]))
        ldy_pad = int(rng.choice([0, 0, 5]))
        alpha = float(rng.choice([1.0, -1.0, 2.0, 0.5]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -0.5]))
        out.append((i, batch, C, H, W, M, R, S, sh, sw, ph, pw, ldw_pad, ldy_pad, alpha, beta))
    return out


CASES = _cases()


def _ints(shape, rng):
    return rng.integers(-3, 4, size=shape).astype(np.float32)


@pytest.mark.parametrize("chunk", range(6))
def test_random_convolutions_integer_exact(chunk):
    import fp32_gemm_04_amd as sg
    stream = torch.cuda.current_stream()
    for case in CASES[chunk::6]:
        i, batch, C, H, W, M, R, S, sh, sw, ph, pw, ldw_pad, ldy_pad, alpha, beta = case
        OH = (H + 2 * ph - R) // sh + 1
        OW = (W + 2 * pw - S) // sw + 1
        N = batch * OH * OW
        K = C * R * S
        rng = np.random.default_rng(1000 + i)
        X = _ints((batch, C, H, W), rng)
        Wt = _ints((M, K), rng)
        Y0 = _ints((M, N), rng)
        ref, _ = oracle.conv2d(X, Wt, R, S, (sh, sw), (ph, pw), Y=Y0, alpha=alpha, beta=beta,
                               with_absdot=False)
        ldw, ldy = K + ldw_pad, N + ldy_pad
        dX = torch.from_numpy(X).cuda()
        wbuf = np.full((M, ldw), np.nan, np.float32)
        wbuf[:, :K] = Wt
        dW = torch.from_numpy(wbuf).cuda()
        for v in FORMS:
            rc, plan = sg.sconv2d_plan(v, batch, C, H, W, M, R, S, sh, sw, ph, pw, 256)
            if rc != 0:
                assert rc == sg.SGEMM_ERR_VARIANT_SHAPE, (case, v, rc)
                continue
            ybuf = np.full((M, ldy), np.nan, np.float32)
            ybuf[:, :N] = Y0
            dY = torch.from_numpy(ybuf).cuda()
            say("conv case %d form %d: %s" % (i, v, plan))
            rc = sg.sconv2d_f32_variant(v, batch, C, H, W, M, R, S, sh, sw, ph, pw, alpha,
                                        dX.data_ptr(), dW.data_ptr(), ldw, beta, dY.data_ptr(),
                                        ldy, stream.cuda_stream)
            if v in (4, 5) and rc == sg.SGEMM_ERR_VARIANT_SHAPE:
                continue  # the plan assumes packed filters; the padded rows are not aligned
            assert rc == 0, (case, v, sg.sgemm_status_string(rc))
            stream.synchronize()
            got = dY.cpu().numpy()
            assert_bits_equal(got[:, :N], ref, "conv case %d form %d (%s)" % (i, v, plan))
            if ldy_pad:
                assert np.all(np.isnan(got[:, N:])), "Y written past its window"
