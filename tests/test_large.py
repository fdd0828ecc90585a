"""Operands beyond 2^31 elements (and a skinny B beyond 2^32 bytes): every
kernel forms addresses in 64 bits, and the skinny kernel's 32-bit fast path
is not taken when offsets would not fit.  Integer data, so sampled rows or
columns must match the reference bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


# (variant, M, N, K, what is large, sampled axis); variant 17 is the 128 x 128
# tile, which takes the direct-load path here.
CASES = [
    (0, 8, 1 << 20, 2100, "B, register-staged path", "cols"),
    (17, 128, 1 << 20, 2112, "B, direct-load path", "cols"),
    (0, 1 << 20, 16, 2112, "A", "rows"),
    (0, 64, 8_000_000, 147, "B over 2^32 bytes, skinny kernel", "cols"),
]


@pytest.mark.parametrize("variant,M,N,K,what,axis", CASES, ids=[c[4] for c in CASES])
def test_beyond_32_bit_indices(variant, M, N, K, what, axis):
    import fp32_gemm_04_amd as sg
    _, plan = sg.sgemm_plan(variant, M, N, K, K, N, N, 1.0, 256)
    say("large operands (%s): M=%d N=%d K=%d plan %s" % (what, M, N, K, plan))
    if "skinny" in what:
        assert plan.startswith("skinny") and " fast=0x" in plan, plan
    if "direct" in what:
        assert " load=direct " in plan, plan
    A = workloads.device_integers(M, K, 970 + K)
    B = workloads.device_integers(K, N, 971 + K)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = sg.sgemm_f32_variant(variant, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0,
                              C.data_ptr(), N, s.cuda_stream)
    assert rc == 0, sg.sgemm_status_string(rc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(972)
    if axis == "cols":
        idx = np.sort(rng.choice(N, 48, replace=False))
        idx[-1] = N - 1
        ref, _ = oracle.sgemm(A.cpu().numpy(), B[:, idx].cpu().numpy(), None, 1.0, 0.0)
        got = C[:, idx].cpu().numpy()
    else:
        idx = np.sort(rng.choice(M, 48, replace=False))
        idx[-1] = M - 1
        ref, _ = oracle.sgemm(A[idx, :].cpu().numpy(), B.cpu().numpy(), None, 1.0, 0.0)
        got = C[idx, :].cpu().numpy()
    assert_bits_equal(got, ref, what)
    del A, B, C
    torch.cuda.empty_cache()


# Stem convolutions whose input passes 2^31 bytes (3600 images of 3 x 224 x
# 224): too large for the stem's buffer-load window fetch, so the aligned
# input is read with plain 128-bit loads from clamped addresses; the output
# (20 x 45 M floats, 3.6 GB) stays under the stem's 4 GiB bound.  Integer
# data drawn on the device; the first, a middle and the last image are
# compared in full with the reference convolution of that image alone.
STEM_LARGE = [(3, 1), (7, 3)]  # (filter size, padding), stride 2


@pytest.mark.parametrize("R,pad", STEM_LARGE, ids=["3x3", "7x7"])
def test_stem_input_beyond_2gib(R, pad):
    import fp32_gemm_04_amd as sg
    batch, C, H, W, M = 3600, 3, 224, 224, 20
    geom = (batch, C, H, W, M, R, R, 2, 2, pad, pad)
    OH = (H + 2 * pad - R) // 2 + 1
    OW = (W + 2 * pad - R) // 2 + 1
    N, K = batch * OH * OW, C * R * R
    assert 4 * batch * C * H * W > 1 << 31
    _, plan = sg.sconv2d_plan(0, *geom, 256)
    say("large stem input: %dx%d, plan %s" % (R, R, plan))
    assert plan.startswith("stem mb=1"), plan
    X = workloads.device_integers(batch * C * H, W, 980 + R)
    Wt = workloads.integers(M, K, 981 + R)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dW = torch.from_numpy(Wt).cuda()
    s = torch.cuda.current_stream()
    rc = sg.sconv2d_f32(*geom, 1.0, X.data_ptr(), dW.data_ptr(), K, 0.0, Y.data_ptr(), N,
                        s.cuda_stream)
    assert rc == 0, sg.sgemm_status_string(rc)
    torch.cuda.synchronize()
    ohw = OH * OW
    for b in (0, batch // 2, batch - 1):
        img = X[b * C * H:(b + 1) * C * H].reshape(1, C, H, W).cpu().numpy()
        ref, _ = oracle.conv2d(img, Wt, R, R, (2, 2), (pad, pad), with_absdot=False)
        got = Y[:, b * ohw:(b + 1) * ohw].cpu().numpy()
        assert_bits_equal(got, ref, "stem %dx%d image %d" % (R, R, b))
    del X, Y
    torch.cuda.empty_cache()
