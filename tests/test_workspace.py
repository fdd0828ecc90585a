"""sgemm_f32 allocates nothing: stream-K partial tiles go to a static device
array the library holds per device.  The first stream-K call on a fresh
stream leaves the device's free memory unchanged, and two stream-K calls in a
row on that stream, the second smaller, each equal the CPU reference bit for
bit (integer data)."""
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


# Both shapes run stream-K with split tiles (partials in the workspace):
# the eight-wave 128 x 128 tile (32 MiB of partials), then the 64 x 64 ring.
SHAPES = [(1280, 1280, 1280), (384, 1000, 2048)]


def _case(i, M, N, K):
    A = workloads.integers(M, K, 990 + 10 * i)
    B = workloads.integers(K, N, 991 + 10 * i)
    ref, _ = oracle.sgemm(A, B)
    return torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), ref


def test_streamk_calls_allocate_nothing():
    import fp32_gemm_04_amd as sg
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cases = []
    for i, (M, N, K) in enumerate(SHAPES):
        plan = sg.sgemm_plan(0, M, N, K, K, N, N, 1.0, cus)[1]
        assert "streamk=0" not in plan and " ws=0" not in plan, plan
        dA, dB, ref = _case(i, M, N, K)
        cases.append((M, N, K, dA, dB, ref, torch.empty((M, N), device="cuda")))
    # Every kernel and HIP resource the calls use exists before measuring:
    # the same calls once on another stream, and the fresh stream's queue.
    warm = torch.cuda.Stream()
    for M, N, K, dA, dB, ref, C in cases:
        say("workspace: warm-up M=%d N=%d K=%d" % (M, N, K))
        assert sg.sgemm_f32(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(),
                            N, warm.cuda_stream) == 0
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for *_, C in cases:
            C.fill_(float("nan"))
    torch.cuda.synchronize()
    free_before, _ = torch.cuda.mem_get_info()
    for M, N, K, dA, dB, ref, C in cases:
        say("workspace: fresh stream M=%d N=%d K=%d" % (M, N, K))
        rc = sg.sgemm_f32(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N,
                          s.cuda_stream)
        assert rc == 0, sg.sgemm_status_string(rc)
    s.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    for M, N, K, dA, dB, ref, C in cases:
        assert_bits_equal(C.cpu().numpy(), ref, "M=%d N=%d K=%d" % (M, N, K))
    assert free_after == free_before, "device free memory changed by %d bytes" % (
        free_before - free_after)
