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
