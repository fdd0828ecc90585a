"""Streams and threads: stream-K calls on different streams never share
partial tiles (each stream holds one of the library's workspace slots, taken
over only once its last use has completed), a slot serves calls of any size
on its stream, and concurrent calls from two host threads give the same bits
as the same calls made one at a time.  Stream-K sums partial tiles in a fixed
order, so every comparison here is bit for bit."""
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


def test_one_slot_serves_every_size_on_its_stream():
    """Stream-K calls with small tiles, then larger ones, then the small ones
    again, queued on one fresh stream without synchronising: each result
    matches the reference."""
    import fp32_gemm_04_amd as sg
    s = torch.cuda.Stream()
    jobs = []
    for i, (variant, M, N, K) in enumerate([(53, 160, 300, 640), (49, 480, 1000, 1280),
                                            (53, 160, 300, 640)]):
        A, B, C = _operands(M, N, K, 820 + 10 * i)
        Cin = C.cpu().numpy()
        say("one stream, step %d: variant %d M=%d N=%d K=%d" % (i, variant, M, N, K))
        _launch(sg, variant, A, B, C, 0.5, -1.0, s)
        jobs.append((A, B, C, Cin))
    s.synchronize()
    for i, (A, B, C, Cin) in enumerate(jobs):
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


def _int_operands(M, N, K, seed):
    A = workloads.integers(M, K, seed)
    B = workloads.integers(K, N, seed + 1)
    return A, B, torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()


def test_more_streams_than_slots_auto():
    """A shape the selector runs stream-K, called on 20 streams in turn (twice
    round) without synchronising: the library holds four workspace slots per
    device, so streams that find them all busy run one tile per workgroup.
    On integer data every plan gives the reference's bits."""
    import fp32_gemm_04_amd as sg
    M, N, K = 384, 3000, 1152
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = sg.sgemm_plan(0, M, N, K, K, N, N, 1.0, cus)[1]
    assert " ws=0" not in plan and "streamk=0" not in plan, plan
    A, B, dA, dB = _int_operands(M, N, K, 860)
    ref, _ = oracle.sgemm(A, B)
    streams = [torch.cuda.Stream() for _ in range(20)]
    outs = [torch.full((M, N), float("nan"), device="cuda") for _ in streams]
    say("AUTO stream-K shape on 20 streams, two rounds")
    for _ in range(2):
        for s, C in zip(streams, outs):
            _launch(sg, 0, dA, dB, C, 1.0, 0.0, s)
    torch.cuda.synchronize()
    for i, C in enumerate(outs):
        assert_bits_equal(C.cpu().numpy(), ref, "stream %d" % i)


def test_forced_streamk_without_free_slot():
    """A forced stream-K variant either runs (a slot was free or idle) or
    returns SGEMM_ERR_NO_SLOT having queued nothing; once the device is idle,
    a call on yet another stream takes an idle slot over and runs."""
    import fp32_gemm_04_amd as sg
    variant, M, N, K = 49, 384, 1000, 1152
    A, B, dA, dB = _int_operands(M, N, K, 870)
    ref, _ = oracle.sgemm(A, B)
    streams = [torch.cuda.Stream() for _ in range(8)]
    outs = [torch.full((M, N), float("nan"), device="cuda") for _ in streams]
    say("forced stream-K on 8 streams without synchronising")
    codes = []
    for s, C in zip(streams, outs):
        codes.append(sg.sgemm_f32_variant(variant, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(),
                                          N, 0.0, C.data_ptr(), N, s.cuda_stream))
    torch.cuda.synchronize()
    assert set(codes) <= {0, sg.SGEMM_ERR_NO_SLOT}, codes
    assert codes[:4].count(0) >= 1
    for i, (rc, C) in enumerate(zip(codes, outs)):
        got = C.cpu().numpy()
        if rc == 0:
            assert_bits_equal(got, ref, "stream %d" % i)
        else:
            assert np.isnan(got).all(), "stream %d: a refused call wrote C" % i
    s = torch.cuda.Stream()
    C = torch.full((M, N), float("nan"), device="cuda")
    say("forced stream-K on a ninth stream after the device went idle")
    rc = sg.sgemm_f32_variant(variant, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                              C.data_ptr(), N, s.cuda_stream)
    assert rc == 0, sg.sgemm_status_string(rc)
    s.synchronize()
    assert_bits_equal(C.cpu().numpy(), ref, "ninth stream")


def test_forced_streamk_beyond_a_slot_refuses():
    """A forced stream-K plan whose partial tiles exceed a workspace slot (the
    160 x 160 tile shared over 512 workers: 100 MiB) returns
    SGEMM_ERR_WORKSPACE and queues nothing; sgemm_plan reports its bytes."""
    import fp32_gemm_04_amd as sg
    M, N, K = 480, 1000, 1280
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = sg.sgemm_plan(48, M, N, K, K, N, N, 1.0, cus)[1]
    ws = int(dict(kv.split("=") for kv in plan.split()[1:])["ws"])
    assert ws > 64 << 20, plan
    A, B, dA, dB = _int_operands(M, N, K, 880)
    C = torch.full((M, N), float("nan"), device="cuda")
    say("forced 160 x 160 stream-K beyond a slot")
    rc = sg.sgemm_f32_variant(48, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                              C.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    assert rc == sg.SGEMM_ERR_WORKSPACE, rc
    torch.cuda.synchronize()
    assert np.isnan(C.cpu().numpy()).all()
