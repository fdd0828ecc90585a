"""GPU parity: libsgemm against the CPU reference, element by element.

Every output element of every workload is compared with the reference's own
value for it: the small and medium shapes, every point of the square sweep
(5120^3 included) and the six im2col shapes at their full sizes, each on
uniform and on integer data.  Integer-valued inputs must match bit for bit;
uniform inputs must satisfy
|gpu - ref| <= 1e-5 * (|alpha| * sum_k |a_ik b_kj| + |beta c_ij|) + 1e-6.
Bytes of C outside its M x N window must keep their NaN guard values.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import assert_bits_equal, assert_within_tolerance, run, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_gemm_04_amd  # noqa: F401  (fails loudly if the library is missing)


def _fits(variant, M, K):
    """The forced skinny kernel only takes M <= 64 and K <= 240."""
    return variant != 3 or (M <= 64 and K <= 240)


def _full_check(A, B, C, alpha, beta, variant=0, exact=False, **kw):
    if not _fits(variant, A.shape[0], A.shape[1]):
        return None
    out, dC = run(A, B, C, alpha, beta, variant=variant, **kw)
    ref, t = oracle.sgemm(A, B, C, alpha, beta)
    if exact:
        assert_bits_equal(out, ref, "variant %d" % variant)
    else:
        assert_within_tolerance(out, ref, t, alpha, beta, C, "variant %d" % variant)
    assert dC.outside_is_nan(), "C written outside its M x N window"
    return out


# AUTO, MFMA (the tile kernel, tile chosen by shape), VALU, SKINNY, the
# forced MFMA tiles, the same tiles run
# stream-K (variant 48 + i), and the eight rungs of the pages' SIMT ladder
# (variant 32 + r).
NUM_TILES = 13  # entries of the MFMA tile table (checked against the library in test_abi)
STREAMK_FAMILIES = [48 + i for i in range(NUM_TILES)]
FAMILIES = ([0, 1, 2, 3] + [16 + i for i in range(NUM_TILES)] + STREAMK_FAMILIES
            + [32 + r for r in range(8)])


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
@pytest.mark.parametrize("variant", FAMILIES)
def test_square256(variant, integer):
    case = workloads.SMALL
    A, B, C = workloads.operands(case, integer)
    _full_check(A, B, C, case.alpha, case.beta, variant, exact=integer)


@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
def test_square1024_with_c_preloaded(integer):
    case = workloads.SQUARE1024
    A, B, C = workloads.operands(case, integer)
    assert C is not None
    _full_check(A, B, C, case.alpha, case.beta, exact=integer)


def _full_size_case(case, integer):
    """The whole M x N output of a workload against the reference's."""
    A, B, C = workloads.operands(case, integer)
    out, dC = run(A, B, C, case.alpha, case.beta, name=case.name)
    ref, t = oracle.sgemm(A, B, C, case.alpha, case.beta, with_absdot=not integer)
    if integer:
        assert_bits_equal(out, ref, case.name)
        say("%s integer: %d elements bit for bit" % (case.name, out.size))
    else:
        worst = assert_within_tolerance(out, ref, t, case.alpha, case.beta, C, case.name)
        say("%s uniform: %d elements, max err/tol %.3g" % (case.name, out.size, worst))
    assert dC.outside_is_nan(), "C written outside its M x N window"


@pytest.mark.parametrize("case", workloads.SWEEP, ids=[c.name for c in workloads.SWEEP])
def test_square_sweep_uniform(case):
    _full_size_case(case, integer=False)


@pytest.mark.parametrize("case", workloads.SWEEP, ids=[c.name for c in workloads.SWEEP])
def test_square_sweep_integer(case):
    # Exact for every n: partial sums of products of [-4, 4] integers stay
    # below 2^24 even at K = 5120, and 1.5x + 0.5c is dyadic.
    _full_size_case(case, integer=True)


@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
@pytest.mark.parametrize("case", workloads.SKINNY + workloads.MID,
                         ids=[c.name for c in workloads.SKINNY + workloads.MID])
def test_im2col_shapes(case, integer):
    _full_size_case(case, integer)


def test_im2col_shape_full_compare_small_n():
    """The mid and skinny shapes' K and M with a short N, compared in full."""
    for M, N, K in [(32, 3001, 27), (64, 2051, 147), (384, 1417, 1152), (256, 777, 1024)]:
        A = workloads.uniform(M, K, M + K)
        B = workloads.uniform(K, N, N + K)
        _full_check(A, B, None, 1.0, 0.0)
        Ai = workloads.integers(M, K, M + K)
        Bi = workloads.integers(K, N, N + K)
        _full_check(Ai, Bi, None, 1.0, 0.0, exact=True)


# ---------------------------------------------------------------- edges

EDGE_SHAPES = [
    (1, 1, 1), (1, 7, 3), (5, 1, 2), (2, 3, 1), (3, 5, 7), (16, 16, 16), (17, 33, 31),
    (31, 17, 65), (33, 65, 33), (63, 64, 127), (65, 63, 129), (127, 129, 5), (129, 127, 257),
    (160, 160, 32), (161, 159, 33), (255, 257, 48), (257, 255, 97), (320, 160, 64),
    (333, 517, 259), (64, 1000, 27), (32, 999, 147), (400, 3, 300), (3, 400, 300),
]


@pytest.mark.parametrize("variant", FAMILIES)
def test_edge_shapes_integer_exact(variant):
    for M, N, K in EDGE_SHAPES:
        A = workloads.integers(M, K, 3 * M + K)
        B = workloads.integers(K, N, 5 * N + K)
        C = workloads.integers(M, N, 7 * M + N)
        _full_check(A, B, C, 1.5, 0.5, variant, exact=True)


@pytest.mark.parametrize("variant", FAMILIES)
def test_edge_shapes_uniform(variant):
    for M, N, K in EDGE_SHAPES[::2]:
        A = workloads.uniform(M, K, 11 * M + K)
        B = workloads.uniform(K, N, 13 * N + K)
        _full_check(A, B, None, 1.0, 0.0, variant)


@pytest.mark.parametrize("variant", FAMILIES)
def test_padded_leading_dimensions(variant):
    for (M, N, K), pads in [((70, 90, 50), (3, 5, 7)), ((161, 33, 64), (4, 4, 4)),
                            ((33, 161, 19), (1, 2, 3))]:
        A = workloads.integers(M, K, 1)
        B = workloads.integers(K, N, 2)
        C = workloads.integers(M, N, 3)
        _full_check(A, B, C, -1.0, 2.0, variant, exact=True,
                    lds=(K + pads[0], N + pads[1], N + pads[2]))


# K a multiple of 16 with 16-byte aligned rows (other K below): the 160, 128, 64x256,
# 64x64 ring, eight-wave 128, 192x128, 96x96, 64x32, 96x224 and 128x176 families
# take the direct global -> LDS path, border tiles
# through its clamped and masked copy.  K = 16 .. 64 covers one to
# four slabs (every prologue case of the three-buffer pipeline); K = 80 an
# odd slab count; ldb is rounded up to a multiple of 4 so that ragged N
# still gives aligned B rows.
DIRECT_SHAPES = [(160, 160, 16), (320, 320, 32), (321, 319, 48), (333, 517, 64),
                 (256, 512, 80), (480, 160, 1024)]
DIRECT_FAMILIES = [16, 17, 20, 22, 23, 24, 25, 26, 27, 28, 48, 49, 52, 54, 55, 56, 57]


def _plan_load(variant, M, N, K, lda, ldb, ldc):
    import fp32_gemm_04_amd as sg
    rc, text = sg.sgemm_plan(variant, M, N, K, lda, ldb, ldc, 1.0, 256)
    assert rc == 0
    return dict(kv.split("=") for kv in text.split()[1:]).get("load")


@pytest.mark.parametrize("variant", [0] + DIRECT_FAMILIES)
def test_direct_load_path_integer_exact(variant):
    for M, N, K in DIRECT_SHAPES:
        A = workloads.integers(M, K, 17 * M + K)
        B = workloads.integers(K, N, 19 * N + K)
        C = workloads.integers(M, N, 23 * M + N)
        nb = -(-N // 4) * 4  # B rows 16-byte aligned even for ragged N
        for lds in [(K, nb, N), (K + 8, nb + 4, N + 12)]:
            if variant in DIRECT_FAMILIES:
                assert _plan_load(variant, M, N, K, *lds) == "direct"
            _full_check(A, B, C, 1.5, 0.5, variant, exact=True, lds=lds)


# K not a multiple of 16 on the direct-load path (A rows aligned through
# lda rounded up to a multiple of 4): the last K % 16 columns are one more
# slab, zero-filled past K; K < 16 is that slab alone.  B rows aligned, then
# not (the shifted form on the 128 tiles and the 64 x 64 ring).  Forced
# stream-K runs its register-staged kernels for such K.
K_TAIL_SHAPES = [(160, 160, 17), (321, 319, 50), (64, 64, 3), (130, 263, 1000),
                 (257, 389, 31), (96, 500, 1)]


@pytest.mark.parametrize("variant", [0] + DIRECT_FAMILIES)
def test_direct_load_k_tail_integer_exact(variant):
    for M, N, K in K_TAIL_SHAPES:
        A = workloads.integers(M, K, 67 * M + K)
        B = workloads.integers(K, N, 71 * N + K)
        C = workloads.integers(M, N, 73 * M + N)
        la = -(-K // 4) * 4
        nb = -(-N // 4) * 4
        for lds, boff in [((la, nb, N), 0), ((la + 4, N + 1, N + 2), 3)]:
            if variant in DIRECT_FAMILIES and boff == 0:
                # the stream-K forms take the register-staged path here
                want = "direct" if variant < 48 else "regs"
                assert _plan_load(variant, M, N, K, *lds) == want
            _full_check(A, B, C, 1.5, 0.5, variant, exact=True, lds=lds, offsets=(0, boff, 0))


@pytest.mark.parametrize("variant", DIRECT_FAMILIES)
def test_direct_load_k_tail_uniform(variant):
    for M, N, K in K_TAIL_SHAPES[1::2]:
        A = workloads.uniform(M, K, 79 * M + K)
        B = workloads.uniform(K, N, 83 * N + K)
        C = workloads.uniform(M, N, 89 * M + N)
        _full_check(A, B, C, -0.75, 1.25, variant, lds=(-(-K // 4) * 4, N, N))


@pytest.mark.parametrize("variant", DIRECT_FAMILIES)
def test_direct_load_path_uniform(variant):
    for M, N, K in DIRECT_SHAPES[1::2]:
        A = workloads.uniform(M, K, 29 * M + K)
        B = workloads.uniform(K, N, 31 * N + K)
        C = workloads.uniform(M, N, 37 * M + N)
        _full_check(A, B, C, -0.75, 1.25, variant)


# B rows that are not 16-byte aligned (ldb % 4 != 0 or a B base off
# 16-byte alignment) with A aligned and K % 16 == 0: the 128 x 128, 64 x 256
# and 64 x 64 ring tiles take the shifted direct-load form, whose row misalignment
# d = 0..3 varies from row to row (ldb % 4 = 1, 2, 3) and with the base
# offset.  Border tiles
# (ragged M and N) run the same body with clamped sources and masked stores;
# the NaN padding past each row and matrix shows any clamped value that
# reaches C.
SHIFTED_SHAPES = [(128, 128, 16), (256, 257, 32), (257, 389, 48), (384, 1001, 64),
                  (130, 263, 80), (384, 1041, 320)]
SHIFTED_FAMILIES = [17, 20, 22, 23, 24, 25, 26, 27, 49, 52, 54, 55, 56, 57]


@pytest.mark.parametrize("variant", [0] + SHIFTED_FAMILIES)
def test_shifted_direct_load_integer_exact(variant):
    for M, N, K in SHIFTED_SHAPES:
        A = workloads.integers(M, K, 41 * M + K)
        B = workloads.integers(K, N, 43 * N + K)
        C = workloads.integers(M, N, 47 * M + N)
        for pad, boff in [(1, 0), (2, 1), (3, 3), (0, 2), (5, 0)]:
            ldb = N + pad
            lds = (K, ldb, N + 3)
            if ldb % 4 == 0 and boff == 0:
                continue
            if variant in SHIFTED_FAMILIES and boff == 0:
                assert _plan_load(variant, M, N, K, *lds) == "shifted"
            _full_check(A, B, C, 1.5, 0.5, variant, exact=True, lds=lds,
                        offsets=(0, boff, 0))


@pytest.mark.parametrize("variant", SHIFTED_FAMILIES)
def test_shifted_direct_load_uniform(variant):
    for M, N, K in SHIFTED_SHAPES[1::2]:
        A = workloads.uniform(M, K, 53 * M + K)
        B = workloads.uniform(K, N, 59 * N + K)
        C = workloads.uniform(M, N, 61 * M + N)
        _full_check(A, B, C, -0.75, 1.25, variant, lds=(K, N + 1, N), offsets=(0, 1, 0))


@pytest.mark.parametrize("variant", FAMILIES)
def test_misaligned_bases(variant):
    """Base pointers off 16-byte alignment take the 32-bit load paths."""
    M, N, K = 97, 131, 75
    A = workloads.integers(M, K, 4)
    B = workloads.integers(K, N, 5)
    C = workloads.integers(M, N, 6)
    for offs in [(1, 0, 0), (0, 2, 0), (3, 1, 2), (0, 0, 1)]:
        _full_check(A, B, C, 1.0, 1.0, variant, exact=True, offsets=offs,
                    lds=(K + 1, N + 3, N))


def test_beta_zero_ignores_nan_in_c():
    M, N, K = 130, 70, 40
    A = workloads.integers(M, K, 8)
    B = workloads.integers(K, N, 9)
    C = np.full((M, N), np.nan, np.float32)
    for variant in FAMILIES:
        out = _full_check(A, B, C, 2.0, 0.0, variant, exact=True)
        assert out is None or not np.isnan(out).any()


def test_alpha_zero_and_k_zero_scale_c():
    M, N = 50, 37
    C = workloads.integers(M, N, 10)
    A = np.full((M, 9), np.nan, np.float32)
    B = np.full((9, N), np.nan, np.float32)
    _full_check(A, B, C, 0.0, -0.5, exact=True)
    _full_check(A, B, C, 0.0, 0.0, exact=True)
    A0 = np.zeros((M, 0), np.float32)
    B0 = np.zeros((0, N), np.float32)
    _full_check(A0, B0, C, 1.0, 3.0, exact=True)


def test_page3_constant_case():
    """A = 1, B = 0.01 at 1024^2 (cnblogs matmul_opt.cu demo).

    The page checks its GPU result against a CPU loop that sums in float,
    with an absolute tolerance of 1e-4; that check is repeated here for one
    element's float running sum.  Constant data makes every rounding of a
    float accumulator err the same way, so the result is not within the
    1e-5 relative bound that holds for random data; against the exact value
    (the fp64 reference) it must meet the classic worst-case bound for a
    K-term float sum in any order, gamma_K * sum|a*b| with
    gamma_K = K u / (1 - K u), u = 2^-24."""
    n = 1024
    A = np.ones((n, n), np.float32)
    B = np.full((n, n), np.float32(0.01), np.float32)
    out, _ = run(A, B, None, 1.0, 0.0, name="page3 constant")
    running = np.float32(0.0)
    for _ in range(n):
        running = np.float32(running + np.float32(0.01))
    assert np.max(np.abs(out.astype(np.float64) - float(running))) <= 1e-4
    ref, t = oracle.sgemm(A[:4], B)
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(out[:4].astype(np.float64) - ref) <= gamma * t)


@pytest.mark.parametrize("variant", FAMILIES)
def test_one_hot_rows(variant):
    """A = e_i e_k^T copies row k of B into row i of C: pins row/column indexing
    at tile boundaries."""
    M, N, K = (333, 289, 97) if variant != 3 else (61, 289, 97)
    B = workloads.uniform(K, N, 12)
    for i, k in [(0, 0), (M - 1, K - 1), (59, 31), (33, 48), (40, 49), (31, 96)] + \
            ([(159, 31), (160, 32), (255, 64), (128, 96)] if variant != 3 else []):
        A = np.zeros((M, K), np.float32)
        A[i, k] = 1.0
        out, _ = run(A, B, None, 1.0, 0.0, variant=variant, name="one-hot %d %d" % (i, k))
        expect = np.zeros((M, N), np.float32)
        expect[i] = B[k]
        assert_bits_equal(out, expect, "one-hot (%d, %d)" % (i, k))


def test_skinny_variant_rejects_large_shapes():
    import fp32_gemm_04_amd as sg
    rc, _ = sg.sgemm_plan(3, 65, 100, 10, 10, 100, 100, 1.0, 256)
    assert rc == sg.SGEMM_ERR_VARIANT_SHAPE
    rc, _ = sg.sgemm_plan(3, 64, 100, 241, 241, 100, 100, 1.0, 256)
    assert rc == sg.SGEMM_ERR_VARIANT_SHAPE


# Skinny shapes with M <= 32, N % 64 == 0 and aligned rows take the 16x16x4
# streaming kernel: one or two 16-row blocks; K = 1 .. 240 (partial last
# step, partial last 16-wide chunk); 4100 strips for 2048 resident waves, so
# waves stream across strip boundaries.
STREAM16_SHAPES = [(32, 64, 147), (17, 1024, 27), (32, 4096, 240), (16, 640, 100),
                   (1, 128, 1), (9, 192, 5), (32, 262400, 27), (32, 262400, 147)]


@pytest.mark.parametrize("M,N,K", STREAM16_SHAPES)
def test_stream16_shapes(M, N, K):
    import fp32_gemm_04_amd as sg
    rc, text = sg.sgemm_plan(3, M, N, K, K, N, N, 1.0, 256)
    assert rc == 0 and text.startswith("stream16")
    A = workloads.integers(M, K, M * 11 + K)
    B = workloads.integers(K, N, N * 13 + K)
    C = workloads.integers(M, N, 3 * M + N)
    _full_check(A, B, C, 1.5, -0.5, 3, exact=True)
    _full_check(A, B, C, 1.0, 2.0, 3, exact=True, lds=(K + 5, N + 64, N + 4))
    Au = workloads.uniform(M, K, M * 11 + K)
    Bu = workloads.uniform(K, N, N * 13 + K)
    _full_check(Au, Bu, None, 1.0, 0.0, 3)


SKINNY_SHAPES = [(32, 1, 27), (1, 33, 1), (32, 33, 2), (64, 95, 147), (33, 1000, 27),
                 (64, 4097, 240), (17, 3333, 239), (64, 64, 148), (2, 70, 3)]


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_kernel_shapes(M, N, K):
    A = workloads.integers(M, K, M * 7 + K)
    B = workloads.integers(K, N, N * 3 + K)
    C = workloads.integers(M, N, M + N)
    _full_check(A, B, C, 1.5, -0.5, 3, exact=True)
    Au = workloads.uniform(M, K, M * 7 + K)
    Bu = workloads.uniform(K, N, N * 3 + K)
    _full_check(Au, Bu, None, 1.0, 0.0, 3)


# Stream-K on shapes with many k-slabs per tile and ragged edges: worker
# ranges then start and end inside tiles (partial tiles at both ends, tiles
# split over three or more workers) and edge tiles take the masked body.
STREAMK_SHAPES = [(300, 200, 1000), (513, 257, 333), (160, 320, 2048), (97, 1000, 640)]
SLOT_BYTES = 2 * 512 * 128 * 128 * 4  # one stream-K workspace slot of the library (64 MiB)


def _sk_refused(variant, M, N, K):
    """A forced stream-K plan whose partial tiles exceed a workspace slot
    (a wide tile shared over many workers: 128 x 176 over more than 372) is
    refused with SGEMM_ERR_WORKSPACE, queuing nothing.  Returns True after
    checking that refusal for such a plan, False for a plan that fits."""
    import fp32_gemm_04_amd as sg
    import torch
    _, text = sg.sgemm_plan(variant, M, N, K, K, N, N, 1.0, 256)
    ws = int(text.split(" ws=")[1].split()[0])
    if ws <= SLOT_BYTES:
        return False
    dA = torch.zeros((M, K), device="cuda")
    dB = torch.zeros((K, N), device="cuda")
    dC = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.current_stream()
    rc = sg.sgemm_f32_variant(variant, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                              dC.data_ptr(), N, s.cuda_stream)
    assert rc == sg.SGEMM_ERR_WORKSPACE, (variant, M, N, K, rc)
    s.synchronize()
    assert torch.isnan(dC).all(), "a refused call wrote C"
    return True


@pytest.mark.parametrize("variant", STREAMK_FAMILIES)
def test_streamk_integer_exact(variant):
    for M, N, K in STREAMK_SHAPES:
        if _sk_refused(variant, M, N, K):
            continue
        A = workloads.integers(M, K, 41 * M + K)
        B = workloads.integers(K, N, 43 * N + K)
        C = workloads.integers(M, N, 47 * M + N)
        _full_check(A, B, C, 1.5, 0.5, variant, exact=True)
        _full_check(A, B, None, 1.0, 0.0, variant, exact=True)


@pytest.mark.parametrize("variant", STREAMK_FAMILIES)
def test_streamk_uniform_repeatable(variant):
    """Uniform data within tolerance, and the same bits on a second call
    (the partial tiles are added in a fixed order)."""
    M, N, K = 513, 257, 333
    assert not _sk_refused(variant, M, N, K)
    A = workloads.uniform(M, K, 53)
    B = workloads.uniform(K, N, 59)
    C = workloads.uniform(M, N, 61)
    first = _full_check(A, B, C, -0.75, 1.25, variant)
    second = _full_check(A, B, C, -0.75, 1.25, variant)
    assert np.array_equal(first.view(np.uint32), second.view(np.uint32))


# The vector-FMA kernel's 160 x 160 tile: shapes where it leaves less work per
# resident workgroup than the 128 tile (529 tiles of 128 over 512 slots
# against 361 of 160), with ragged edges and K not a multiple of 8.
VALU160_SHAPES = [(2900, 2900, 40), (3000, 2800, 37)]


@pytest.mark.parametrize("M,N,K", VALU160_SHAPES)
def test_valu_160_tile_integer_exact(M, N, K):
    import fp32_gemm_04_amd as sg
    _, text = sg.sgemm_plan(sg.SGEMM_VARIANT_VALU, M, N, K, K, N, N, 1.0, 256)
    assert " bm=160 " in text, text
    A = workloads.integers(M, K, 900 + K)
    B = workloads.integers(K, N, 901 + K)
    C = workloads.integers(M, N, 902 + K)
    _full_check(A, B, C, 1.0, -2.0, variant=sg.SGEMM_VARIANT_VALU, exact=True)


@pytest.mark.parametrize("M,N,K", VALU160_SHAPES)
def test_valu_160_tile_uniform(M, N, K):
    import fp32_gemm_04_amd as sg
    A = workloads.uniform(M, K, 910 + K)
    B = workloads.uniform(K, N, 911 + K)
    C = workloads.uniform(M, N, 912 + K)
    _full_check(A, B, C, 1.5, 0.5, variant=sg.SGEMM_VARIANT_VALU)
