"""HIP graph capture: sgemm_f32 launches only kernels on the caller's stream
(no copies, no memsets, no allocation, no event records under capture), so it
can be captured into a graph and replayed.  Each replay, with eager work of
the program and synchronisations between replays, must give the same bits as
an eager call of the captured plan.

Under capture the library never hands a graph a pointer into its stream-K
workspace (a replay may run on any stream at any time): a shape the selector
runs stream-K is captured one tile per workgroup, and a forced stream-K
variant refuses with SGEMM_ERR_CAPTURING.  Those cases use integer data, on
which every plan gives the reference's bits."""
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


def _call(sg, variant, M, N, K, alpha, beta, A, B, C, stream):
    return sg.sgemm_f32_variant(variant, M, N, K, alpha, A.data_ptr(), K, B.data_ptr(), N,
                                beta, C.data_ptr(), N, stream.cuda_stream)


def _replays_match(sg, variant, M, N, K, alpha, beta, A, B, C0, ref, fresh_stream):
    """Capture one call on a side stream, replay it four times with eager
    calls between, and compare every result with `ref` (a host array)."""
    s = torch.cuda.Stream()
    C = C0.clone()
    if not fresh_stream:
        with torch.cuda.stream(s):  # warm-up on the capture stream
            assert _call(sg, variant, M, N, K, alpha, beta, A, B, C, s) == 0
        s.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph: capture variant %d M=%d N=%d K=%d" % (variant, M, N, K))
    with torch.cuda.graph(graph, stream=s):
        rc = _call(sg, variant, M, N, K, alpha, beta, A, B, C, torch.cuda.current_stream())
    assert rc == 0, sg.sgemm_status_string(rc)
    other = torch.empty_like(C0)
    for r in range(4):
        C.copy_(C0)
        torch.cuda.synchronize()
        say("graph: replay %d" % r)
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(C.cpu().numpy(), ref, "replay %d" % r)
        # Eager work of the program between replays, on the library too.
        other.copy_(C0)
        assert _call(sg, variant, M, N, K, alpha, beta, A, B, other,
                     torch.cuda.current_stream()) == 0
        torch.cuda.synchronize()
        assert_bits_equal(other.cpu().numpy(), ref, "eager after replay %d" % r)


# (variant, M, N, K, alpha, beta): one tile per workgroup, a forced tile,
# the skinny streaming kernel, and odd N (B rows unaligned: the shifted
# direct-load form, with border tiles).  Uniform data: the eager call runs
# the captured plan, so the bits must agree.
CASES = [(0, 640, 768, 512, 1.5, 0.5), (17, 384, 1000, 1152, 1.0, -1.0),
         (0, 64, 163840, 147, 1.0, 0.0), (0, 384, 2001, 320, 1.0, 0.5)]


@pytest.mark.parametrize("variant,M,N,K,alpha,beta", CASES,
                         ids=["tile", "forced_tile", "skinny", "shifted"])
def test_captured_call_replays_like_eager(variant, M, N, K, alpha, beta):
    import fp32_gemm_04_amd as sg
    A = torch.from_numpy(workloads.uniform(M, K, 950 + K)).cuda()
    B = torch.from_numpy(workloads.uniform(K, N, 951 + K)).cuda()
    C0 = torch.from_numpy(workloads.uniform(M, N, 952 + K)).cuda()
    ref = C0.clone()
    say("graph: eager reference, variant %d M=%d N=%d K=%d" % (variant, M, N, K))
    assert _call(sg, variant, M, N, K, alpha, beta, A, B, ref, torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    _replays_match(sg, variant, M, N, K, alpha, beta, A, B, C0, ref.cpu().numpy(), False)


# Shapes the selector runs stream-K on aligned operands (the 64 x 64 ring,
# the eight-wave 128 x 128 tile) and with B rows unaligned (shifted form).
STREAMK_SHAPES = [(384, 1000, 2048, 1.0, 0.0), (1280, 1280, 1280, 1.5, 0.5),
                  (384, 2001, 1152, -1.0, 1.0)]


@pytest.mark.parametrize("M,N,K,alpha,beta", STREAMK_SHAPES, ids=["ring", "eight_wave", "shifted"])
def test_first_streamk_call_on_fresh_stream_captured(M, N, K, alpha, beta):
    """The first call of a stream-K shape on a fresh stream is made under
    capture; its replays equal the CPU reference bit for bit."""
    import fp32_gemm_04_amd as sg
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = sg.sgemm_plan(0, M, N, K, K, N, N, alpha, cus)[1]
    assert "streamk=0" not in plan and " ws=0" not in plan, plan
    A = workloads.integers(M, K, 960 + K)
    B = workloads.integers(K, N, 961 + K)
    C = workloads.integers(M, N, 962 + K)
    ref, _ = oracle.sgemm(A, B, C, alpha, beta)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (A, B, C))
    _replays_match(sg, 0, M, N, K, alpha, beta, dA, dB, dC0, ref, True)


def test_forced_streamk_refuses_capture():
    """A forced stream-K variant under capture returns SGEMM_ERR_CAPTURING and
    queues nothing; the capture stays usable."""
    import fp32_gemm_04_amd as sg
    M, N, K = 384, 1000, 1152
    A = torch.from_numpy(workloads.integers(M, K, 970)).cuda()
    B = torch.from_numpy(workloads.integers(K, N, 971)).cuda()
    C = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    say("graph: forced stream-K under capture")
    with torch.cuda.graph(graph, stream=s):
        rc = _call(sg, 49, M, N, K, 1.0, 0.0, A, B, C, torch.cuda.current_stream())
        rc2 = _call(sg, 17, M, N, K, 1.0, 0.0, A, B, C, torch.cuda.current_stream())
    assert rc == sg.SGEMM_ERR_CAPTURING, rc
    assert rc2 == 0, sg.sgemm_status_string(rc2)
    graph.replay()
    torch.cuda.synchronize()
    ref, _ = oracle.sgemm(A.cpu().numpy(), B.cpu().numpy())
    assert_bits_equal(C.cpu().numpy(), ref, "forced tile captured after the refusal")
    assert not np.isnan(C.cpu().numpy()).any()
