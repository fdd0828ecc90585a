"""sgemm_tune on the GPU: the tuning call computes C like sgemm_f32, records a
valid variant, and later sgemm_f32 calls with the same key launch exactly
that variant (bit-identical to forcing it), until sgemm_tune_reset."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import DevMat, assert_bits_equal, assert_within_tolerance, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu_and_empty_table():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd as sg
    sg.sgemm_tune_reset()
    yield
    sg.sgemm_tune_reset()


def _valid_variants():
    import fp32_gemm_04_amd as sg
    n = sg.sgemm_num_mfma_tiles()
    return ({sg.SGEMM_VARIANT_AUTO, sg.SGEMM_VARIANT_SKINNY}
            | set(range(sg.SGEMM_VARIANT_MFMA_TILE, sg.SGEMM_VARIANT_MFMA_TILE + n))
            | set(range(sg.SGEMM_VARIANT_STREAMK_TILE, sg.SGEMM_VARIANT_STREAMK_TILE + n)))


# (M, N, K, alpha, beta, float offsets of A, B, C from a 16-byte boundary)
SHAPES = [
    (512, 512, 512, 1.5, 0.5, (0, 0, 0)),     # small square: one tile per CU
    (64, 8192, 147, 1.0, 0.0, (0, 0, 0)),     # skinny, K not a multiple of any slab
    (96, 1001, 64, 1.0, 0.5, (0, 0, 0)),      # odd N: register-staged path
    (256, 1536, 1152, 1.0, 0.0, (0, 0, 0)),   # a slice of the mid im2col shapes
    (200, 328, 96, -0.75, 2.0, (0, 0, 1)),    # C off a 16-byte boundary
]
IDS = ["%dx%dx%d" % s[:3] for s in SHAPES]


def _tune(sg, A, B, C, alpha, beta, offsets, reps=2):
    M, K = A.shape
    N = B.shape[1]
    dA, dB, dC = DevMat(A, offset=offsets[0]), DevMat(B, offset=offsets[1]), DevMat(C, offset=offsets[2])
    s = torch.cuda.current_stream()
    say("sgemm_tune M=%d N=%d K=%d alpha=%g beta=%g offsets=%s" % (M, N, K, alpha, beta, offsets))
    rc, chosen, us = sg.sgemm_tune(M, N, K, alpha, dA.ptr, dA.ld, dB.ptr, dB.ld, beta, dC.ptr,
                                   dC.ld, s.cuda_stream, reps)
    torch.cuda.synchronize()
    assert rc == 0, sg.sgemm_status_string(rc)
    return dA, dB, dC, chosen, us


def _call(sg, variant, dA, dB, C, alpha, beta, offset):
    M, N, K = C.shape[0], C.shape[1], dA.cols
    dC = DevMat(C, offset=offset)
    s = torch.cuda.current_stream()
    say("sgemm variant=%d M=%d N=%d K=%d after tuning" % (variant, M, N, K))
    rc = sg.sgemm_f32_variant(variant, M, N, K, alpha, dA.ptr, dA.ld, dB.ptr, dB.ld, beta,
                              dC.ptr, dC.ld, s.cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0, sg.sgemm_status_string(rc)
    assert dC.outside_is_nan(), "C written outside its window"
    return dC.window()


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_tune_integer_exact(shape):
    """Integer data: the tuning call's own result, and sgemm_f32's after it,
    match the reference bit for bit; the plan names the tuned variant."""
    import fp32_gemm_04_amd as sg
    M, N, K, alpha, beta, offsets = shape
    A = workloads.integers(M, K, 700 + M)
    B = workloads.integers(K, N, 701 + N)
    C = workloads.integers(M, N, 702 + K)
    ref, _ = oracle.sgemm(A, B, C, alpha, beta)
    dA, dB, dC, chosen, us = _tune(sg, A, B, C, alpha, beta, offsets)
    assert chosen in _valid_variants() and us > 0.0
    assert_bits_equal(dC.window(), ref, "tuning call (chose %d)" % chosen)
    assert dC.outside_is_nan(), "tuning wrote C outside its window"
    assert_bits_equal(_call(sg, 0, dA, dB, C, alpha, beta, offsets[2]), ref, "after tuning")
    if offsets == (0, 0, 0):
        _, text = sg.sgemm_plan(0, M, N, K, K, N, N, alpha, 256)
        if chosen != sg.SGEMM_VARIANT_AUTO:
            assert text.endswith(" tuned=%d" % chosen), text
        sg.sgemm_tune_reset()
        _, text = sg.sgemm_plan(0, M, N, K, K, N, N, alpha, 256)
        assert "tuned=" not in text


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_tune_routes_auto_to_the_chosen_kernel(shape):
    """Uniform data: after tuning, sgemm_f32 gives the same bits as forcing
    the chosen variant, within tolerance of the reference; after a reset it
    gives the selector's result again."""
    import fp32_gemm_04_amd as sg
    M, N, K, alpha, beta, offsets = shape
    A = workloads.uniform(M, K, 710 + M)
    B = workloads.uniform(K, N, 711 + N)
    C = workloads.uniform(M, N, 712 + K)
    ref, absdot = oracle.sgemm(A, B, C, alpha, beta)
    untuned = _call(sg, 0, DevMat(A, offset=offsets[0]), DevMat(B, offset=offsets[1]), C,
                    alpha, beta, offsets[2])
    dA, dB, dC, chosen, _ = _tune(sg, A, B, C, alpha, beta, offsets)
    assert_within_tolerance(dC.window(), ref, absdot, alpha, beta, C, "tuning call")
    auto = _call(sg, 0, dA, dB, C, alpha, beta, offsets[2])
    forced = _call(sg, chosen, dA, dB, C, alpha, beta, offsets[2])
    assert_bits_equal(auto, forced, "AUTO after tuning vs variant %d" % chosen)
    assert_bits_equal(dC.window(), forced, "tuning call vs variant %d" % chosen)
    assert_within_tolerance(auto, ref, absdot, alpha, beta, C, "after tuning")
    sg.sgemm_tune_reset()
    assert_bits_equal(_call(sg, 0, dA, dB, C, alpha, beta, offsets[2]), untuned, "after reset")


def test_tune_key_separates_alignment():
    """The same sizes with C off a 16-byte boundary are another key."""
    import fp32_gemm_04_amd as sg
    M, N, K = 64, 8192, 147
    A = workloads.uniform(M, K, 720)
    B = workloads.uniform(K, N, 721)
    C = workloads.uniform(M, N, 722)
    _, _, _, chosen, _ = _tune(sg, A, B, C, 1.0, 0.0, (0, 0, 0))
    _, text_aligned = sg.sgemm_plan(0, M, N, K, K, N, N, 1.0, 256)
    # ldc = N + 1 is another key: nothing tuned for it.
    _, text_other = sg.sgemm_plan(0, M, N, K, K, N, N + 1, 1.0, 256)
    assert "tuned=" not in text_other
    if chosen != sg.SGEMM_VARIANT_AUTO:
        assert "tuned=%d" % chosen in text_aligned


def test_tune_quick_return_records_nothing():
    """K == 0: C <- beta C, no tuning, nothing recorded."""
    import fp32_gemm_04_amd as sg
    M, N = 33, 70
    A = np.zeros((M, 0), np.float32)
    B = np.zeros((0, N), np.float32)
    C = workloads.uniform(M, N, 730)
    dC = DevMat(C)
    s = torch.cuda.current_stream()
    say("sgemm_tune quick return M=%d N=%d K=0" % (M, N))
    rc, chosen, us = sg.sgemm_tune(M, N, 0, 1.0, 0, 1, 0, N, 0.5, dC.ptr, dC.ld, s.cuda_stream, 2)
    torch.cuda.synchronize()
    assert (rc, chosen, us) == (0, sg.SGEMM_VARIANT_AUTO, 0.0)
    ref, _ = oracle.sgemm(A, B, C, 1.0, 0.5)
    assert_bits_equal(dC.window(), ref, "K == 0")
