"""HIP graph capture of the convolution entry points: a call queues kernels
on the caller's stream and nothing else (no copies, memsets, events or
allocation), and the pointwise route's per-image products go through
sgemm_f32, which stays capture-safe on its own.  Each form is captured once
and replayed four times, with eager calls of the library and host
synchronisations between replays; integer data, so every replay must give the
reference convolution's bits."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


# (variant, plan prefix, batch, C, H, W, M, R, S, sh, sw, ph, pw)
CASES = [
    (1, "stem mb=2", 1, 3, 200, 198, 64, 7, 7, 2, 2, 3, 3),
    (1, "stem mb=1", 2, 3, 180, 181, 32, 3, 3, 2, 2, 1, 1),
    (5, "tap", 2, 16, 21, 21, 100, 3, 3, 1, 1, 1, 1),
    (4, "direct", 2, 16, 21, 21, 100, 3, 3, 1, 1, 1, 1),
    (3, "tile", 2, 12, 19, 17, 70, 3, 3, 1, 2, 1, 0),
    (2, "general", 2, 5, 13, 11, 37, 5, 3, 2, 1, 2, 1),
    (0, "gemm images=3", 3, 32, 14, 14, 96, 1, 1, 1, 1, 0, 0),
]


def _launch(sg, v, g, alpha, beta, dX, dW, ldw, dY, ldy, stream):
    batch, C, H, W, M, R, S, sh, sw, ph, pw = g
    return sg.sconv2d_f32_variant(v, batch, C, H, W, M, R, S, sh, sw, ph, pw, alpha,
                                  dX.data_ptr(), dW.data_ptr(), ldw, beta, dY.data_ptr(), ldy,
                                  stream.cuda_stream)


@pytest.mark.parametrize("case", CASES, ids=[c[1].split()[0] + "-%d" % i
                                             for i, c in enumerate(CASES)])
def test_captured_convolution_replays_like_reference(case):
    import fp32_gemm_04_amd as sg
    v, prefix, *g = case
    batch, C, H, W, M, R, S, sh, sw, ph, pw = g
    rc, plan = sg.sconv2d_plan(v, *g, 256)
    assert rc == 0 and plan.startswith(prefix), (rc, plan)
    OH = (H + 2 * ph - R) // sh + 1
    OW = (W + 2 * pw - S) // sw + 1
    N, K = batch * OH * OW, C * R * S
    rng = np.random.default_rng(77 + v)
    X = rng.integers(-3, 4, size=(batch, C, H, W)).astype(np.float32)
    Wt = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    Y0 = rng.integers(-3, 4, size=(M, N)).astype(np.float32)
    alpha, beta = 2.0, -1.0
    ref, _ = oracle.conv2d(X, Wt, R, S, (sh, sw), (ph, pw), Y=Y0, alpha=alpha, beta=beta,
                           with_absdot=False)
    dX, dW = torch.from_numpy(X).cuda(), torch.from_numpy(Wt).cuda()
    dY0 = torch.from_numpy(Y0).cuda()
    dY, other = dY0.clone(), dY0.clone()

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # warm-up on the capture stream
        assert _launch(sg, v, g, alpha, beta, dX, dW, K, dY, N, s) == 0
    s.synchronize()
    dY.copy_(dY0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("conv graph: capture %s" % plan)
    with torch.cuda.graph(graph, stream=s):
        rc = _launch(sg, v, g, alpha, beta, dX, dW, K, dY, N, torch.cuda.current_stream())
    assert rc == 0, sg.sgemm_status_string(rc)
    main = torch.cuda.current_stream()
    for r in range(4):
        dY.copy_(dY0)
        torch.cuda.synchronize()
        say("conv graph: replay %d" % r)
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(dY.cpu().numpy(), ref, "%s replay %d" % (plan, r))
        # eager work of the program, through the library, between replays
        other.copy_(dY0)
        assert _launch(sg, v, g, alpha, beta, dX, dW, K, other, N, main) == 0
        main.synchronize()
        assert_bits_equal(other.cpu().numpy(), ref, "%s eager after replay %d" % (plan, r))
