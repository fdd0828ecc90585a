"""Seeded random problems (960 through every kernel family, then 320 on the
direct-load path): sizes, leading-dimension padding, base misalignment,
alpha and beta drawn at random (one fixed seed, so every run draws the same
cases).  Integer data, so every output must match
the reference bit for bit, and nothing outside C's window may change."""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import assert_bits_equal, run, say
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401


def _families():
    import fp32_gemm_04_amd as sg
    n = sg.sgemm_num_mfma_tiles()
    return ([sg.SGEMM_VARIANT_AUTO, sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU,
             sg.SGEMM_VARIANT_SKINNY]
            + [sg.SGEMM_VARIANT_MFMA_TILE + i for i in range(n)]
            + [sg.SGEMM_VARIANT_STREAMK_TILE + i for i in range(n)]
            + [sg.SGEMM_VARIANT_LADDER + r for r in range(sg.SGEMM_LADDER_RUNGS)])


def _cases(count=960, seed=2024):
    rng = np.random.default_rng(seed)
    fams = _families()
    out = []
    for i in range(count):
        v = fams[i % len(fams)]
        big = rng.random() < 0.3
        M = int(rng.integers(1, 400 if big else 140))
        N = int(rng.integers(1, 400 if big else 140))
        K = int(rng.integers(1, 600 if big else 150))
        if v == 3:  # the skinny kernel takes M <= 64, K <= 240
            M, K = min(M, 64), min(K, 240)
        pads = [int(p) if rng.random() < 0.4 else 0 for p in rng.integers(1, 9, 3)]
        offs = [int(o) if rng.random() < 0.3 else 0 for o in rng.integers(1, 4, 3)]
        alpha = float(rng.choice([1.0, -1.0, 0.5, 1.5, 2.0, 0.0]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -0.5, 0.25]))
        out.append((i, v, M, N, K, pads, offs, alpha, beta))
    return out


CASES = _cases()
SLOT_BYTES = 2 * 512 * 128 * 128 * 4  # one stream-K workspace slot of the library (64 MiB)


def _over_slot(v, M, N, K, lds):
    """A forced stream-K plan whose partial tiles exceed a workspace slot is
    refused with SGEMM_ERR_WORKSPACE (the header's contract, checked in
    test_parity); such a case is skipped here."""
    import fp32_gemm_04_amd as sg
    if v < sg.SGEMM_VARIANT_STREAMK_TILE:
        return False
    rc, text = sg.sgemm_plan(v, M, N, K, lds[0], lds[1], lds[2], 1.0, 256)
    return rc == 0 and " ws=" in text and int(text.split(" ws=")[1].split()[0]) > SLOT_BYTES


@pytest.mark.parametrize("chunk", range(8))
def test_random_problems_integer_exact(chunk):
    for (i, v, M, N, K, pads, offs, alpha, beta) in CASES[chunk::8]:
        A = workloads.integers(M, K, 5000 + 3 * i)
        B = workloads.integers(K, N, 5001 + 3 * i)
        C = workloads.integers(M, N, 5002 + 3 * i)
        lds = (K + pads[0], N + pads[1], N + pads[2])
        if _over_slot(v, M, N, K, lds):
            continue
        say("random case %d: variant %d M=%d N=%d K=%d pads=%s offsets=%s alpha=%g beta=%g"
            % (i, v, M, N, K, pads, offs, alpha, beta))
        out, dC = run(A, B, C, alpha, beta, variant=v, lds=lds, offsets=tuple(offs),
                      name="random %d" % i)
        ref, _ = oracle.sgemm(A, B, C, alpha, beta)
        assert_bits_equal(out, ref, "random case %d (variant %d)" % (i, v))
        assert dC.outside_is_nan(), "case %d: C written outside its window" % i


def _direct_cases(count=320, seed=4096):
    """A rows aligned, so the direct-load kernels run: K a multiple of 16 or
    not (the zero-filled last slab), ragged M and N (border tiles through the
    clamped, masked body), B rows
    at every alignment (the shifted form) and base offsets of B and C."""
    # AUTO and the tile entries that have direct-load kernels (160, 128,
    # 64x256, the 64x64 ring, the eight-wave 128, 192x128, 96x96, 64x32,
    # 96x224, 128x176), one tile per workgroup, and those with direct-load
    # stream-K kernels run stream-K.
    fams = [0, 16, 17, 20, 22, 23, 24, 25, 26, 27, 28, 48, 49, 52, 54, 55, 56, 57]
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        v = fams[i % len(fams)]
        M = int(rng.integers(1, 420))
        N = int(rng.integers(1, 700))
        K = 16 * int(rng.integers(1, 24)) if rng.random() < 0.6 else int(rng.integers(1, 380))
        lda = -(-K // 4) * 4 + 4 * int(rng.integers(0, 3))
        aligned = rng.random() < 0.4  # else the shifted form (on the 128 tiles)
        ldb = (-(-N // 4) * 4 + 4 * int(rng.integers(0, 2))) if aligned else N + int(rng.integers(0, 8))
        ldc = N + int(rng.integers(0, 5))
        offs = [0, 0 if aligned else int(rng.integers(0, 4)), int(rng.integers(0, 4))]
        alpha = float(rng.choice([1.0, -0.5, 2.0]))
        beta = float(rng.choice([0.0, 1.0, -1.5]))
        out.append((i, v, M, N, K, (lda, ldb, ldc), offs, alpha, beta))
    return out


@pytest.mark.parametrize("chunk", range(4))
def test_random_direct_load_problems_integer_exact(chunk):
    for (i, v, M, N, K, lds, offs, alpha, beta) in _direct_cases()[chunk::4]:
        A = workloads.integers(M, K, 9000 + 3 * i)
        B = workloads.integers(K, N, 9001 + 3 * i)
        C = workloads.integers(M, N, 9002 + 3 * i)
        if _over_slot(v, M, N, K, lds):
            continue
        say("direct case %d: variant %d M=%d N=%d K=%d lds=%s offsets=%s alpha=%g beta=%g"
            % (i, v, M, N, K, lds, offs, alpha, beta))
        out, dC = run(A, B, C, alpha, beta, variant=v, lds=lds, offsets=tuple(offs),
                      name="direct %d" % i)
        ref, _ = oracle.sgemm(A, B, C, alpha, beta)
        assert_bits_equal(out, ref, "direct case %d (variant %d)" % (i, v))
        assert dC.outside_is_nan(), "case %d: C written outside its window" % i
