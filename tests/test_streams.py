"""Streams and threads: stream-K calls on different streams use different
workspaces, a workspace grows when a later call needs more, and concurrent
calls from two host threads give the same bits as the same calls made one at
a time.  Stream-K sums partial tiles in a fixed order, so every comparison
here is bit for bit."""
import threading

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


def _operands(M, N, K, seed):
    A = torch.from_numpy(workloads.uniform(M, K, seed)).cuda()
    B = torch.from_numpy(workloads.uniform(K, N, seed + 1)).cuda()
    C = torch.from_numpy(workloads.uniform(M, N, seed + 2)).cuda()
    return A, B, C


def _launch(sg, variant, A, B, C, alpha, beta, stream):
    M, K = A.shape
    N = B.shape[1]
    rc = sg.sgemm_f32_variant(variant, M, N, K, alpha, A.data_ptr(), K, B.data_ptr(), N, beta,
                              C.data_ptr(), N, stream.cuda_stream)
    assert rc == 0, sg.sgemm_status_string(rc)


# (variant, M, N, K): forced stream-K on two tiles, and an AUTO shape that the
# selector runs stream-K (784 tiles of 128 over 512 resident workgroups).
CASES = [(49, 384, 1000, 1152), (50, 200, 700, 2048), (0, 256, 50176, 1024)]


def test_two_streams_concurrently():
    """Two problems, each on its own stream, launched alternately several
    times without synchronising: the results equal one-stream runs."""
    import fp32_gemm_04_amd as sg
    (v1, *s1), (v2, *s2) = CASES[0], CASES[1]
    A1, B1, C1 = _operands(*s1, 800)
    A2, B2, C2 = _operands(*s2, 810)
    ref1, ref2 = C1.clone(), C2.clone()
    main = torch.cuda.current_stream()
    say("one stream: variants %d and %d" % (v1, v2))
    _launch(sg, v1, A1, B1, ref1, 1.0, 0.0, main)
    _launch(sg, v2, A2, B2, ref2, 1.0, 0.0, main)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    say("two streams: variants %d and %d, 6 rounds" % (v1, v2))
    for _ in range(6):
        _launch(sg, v1, A1, B1, C1, 1.0, 0.0, sa)
        _launch(sg, v2, A2, B2, C2, 1.0, 0.0, sb)
    torch.cuda.synchronize()
    assert_bits_equal(C1.cpu().numpy(), ref1.cpu().numpy(), "stream a")
    assert_bits_equal(C2.cpu().numpy(), ref2.cpu().numpy(), "stream b")


def test_workspace_grows_on_one_stream():
    """A stream-K call with small tiles, then one needing a larger workspace,
    then the small one again, on one fresh stream: all match the reference."""
    import fp32_gemm_04_amd as sg
    s = torch.cuda.Stream()
    for i, (variant, M, N, K) in enumerate([(53, 160, 300, 640), (48, 480, 1000, 1280),
                                            (53, 160, 300, 640)]):
        A, B, C = _operands(M, N, K, 820 + 10 * i)
        Cin = C.cpu().numpy()
        say("workspace growth step %d: variant %d M=%d N=%d K=%d" % (i, variant, M, N, K))
        _launch(sg, variant, A, B, C, 0.5, -1.0, s)
        s.synchronize()
        ref, absdot = oracle.sgemm(A.cpu().numpy(), B.cpu().numpy(), Cin, 0.5, -1.0)
        tol = oracle.tolerance(0.5, -1.0, absdot, Cin)
        err = np.abs(C.cpu().numpy().astype(np.float64) - ref.astype(np.float64))
        assert np.all(err <= tol), "step %d: max error %g" % (i, float(np.max(err - tol)))


def test_two_host_threads():
    """Two host threads, each with its own stream, call the library at the
    same time (ctypes releases the interpreter lock during the call)."""
    import fp32_gemm_04_amd as sg
    jobs = []
    for j, (variant, M, N, K) in enumerate([CASES[0], CASES[2]]):
        A, B, C = _operands(M, N, K, 840 + 10 * j)
        ref = C.clone()
        say("thread job %d reference: variant %d" % (j, variant))
        _launch(sg, variant, A, B, ref, 1.0, 0.0, torch.cuda.current_stream())
        jobs.append((variant, A, B, C, ref))
    torch.cuda.synchronize()
    errors = []

    def work(job):
        try:
            variant, A, B, C, _ = job
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    _launch(sg, variant, A, B, C, 1.0, 0.0, s)
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    say("two host threads, 4 calls each")
    threads = [threading.Thread(target=work, args=(job,)) for job in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for j, (_, _, _, C, ref) in enumerate(jobs):
        assert_bits_equal(C.cpu().numpy(), ref.cpu().numpy(), "thread %d" % j)


def test_more_streams_than_kept_workspaces():
    """Stream-K calls on 20 streams in turn (twice round), more than the 16
    workspaces the library keeps per device: later streams take over the
    least recently used ones, after the device has finished the work queued
    on them.  Every result equals the one-stream run."""
    import fp32_gemm_04_amd as sg
    variant, M, N, K = 49, 384, 1000, 1152
    A, B, C0 = _operands(M, N, K, 860)
    ref = C0.clone()
    _launch(sg, variant, A, B, ref, 1.0, 0.0, torch.cuda.current_stream())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(20)]
    outs = [torch.empty_like(C0) for _ in streams]
    say("stream-K on 20 streams, two rounds")
    for _ in range(2):
        for s, C in zip(streams, outs):
            _launch(sg, variant, A, B, C, 1.0, 0.0, s)
    torch.cuda.synchronize()
    for i, C in enumerate(outs):
        assert_bits_equal(C.cpu().numpy(), ref.cpu().numpy(), "stream %d" % i)
