"""HIP graph capture: sgemm_f32 launches only kernels on the caller's stream
(no copies, no memsets, no allocation once a stream's stream-K workspace
exists), so it can be captured into a graph and replayed.  Each replay, with
eager work of the program and synchronisations between replays, must give
the same bits as an eager call."""
import pytest

import workloads
from tests.gpu_helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


# (variant, M, N, K, alpha, beta): one tile per workgroup, stream-K (which
# also launches the fixup kernel), the skinny streaming kernel, and odd N
# (B rows unaligned: the shifted direct-load form, one tile per workgroup
# and stream-K, with border tiles).
CASES = [(0, 640, 768, 512, 1.5, 0.5), (49, 384, 1000, 1152, 1.0, -1.0),
         (0, 64, 163840, 147, 1.0, 0.0), (0, 384, 2001, 320, 1.0, 0.5),
         (55, 384, 2001, 1152, -1.0, 1.0)]


@pytest.mark.parametrize("variant,M,N,K,alpha,beta", CASES,
                         ids=["tile", "streamk", "skinny", "shifted", "shifted_streamk"])
def test_captured_call_replays_like_eager(variant, M, N, K, alpha, beta):
    import fp32_gemm_04_amd as sg
    A = torch.from_numpy(workloads.uniform(M, K, 950 + K)).cuda()
    B = torch.from_numpy(workloads.uniform(K, N, 951 + K)).cuda()
    C0 = torch.from_numpy(workloads.uniform(M, N, 952 + K)).cuda()

    def call(C, stream):
        rc = sg.sgemm_f32_variant(variant, M, N, K, alpha, A.data_ptr(), K, B.data_ptr(), N,
                                  beta, C.data_ptr(), N, stream.cuda_stream)
        assert rc == 0, sg.sgemm_status_string(rc)

    ref = C0.clone()
    say("graph: eager reference, variant %d M=%d N=%d K=%d" % (variant, M, N, K))
    call(ref, torch.cuda.current_stream())
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    C = C0.clone()
    with torch.cuda.stream(s):
        call(C, s)  # warm-up on the capture stream: the stream-K workspace exists before capture
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(graph, stream=s):
        call(C, torch.cuda.current_stream())
    other = torch.empty_like(C0)
    for r in range(4):
        C.copy_(C0)
        torch.cuda.synchronize()
        say("graph: replay %d" % r)
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(C.cpu().numpy(), ref.cpu().numpy(), "replay %d" % r)
        # Eager work of the program between replays, on the library too.
        other.copy_(C0)
        call(other, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert_bits_equal(other.cpu().numpy(), ref.cpu().numpy(), "eager after replay %d" % r)
