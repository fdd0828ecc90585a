"""The C ABI of libsgemm on a host without a GPU: the library loads, exports
every function that include/sgemm.h declares, rejects bad arguments before any
HIP call, reports HIP failures as positive codes, and its tile selector (pure
host logic) picks sensible kernels."""
import ctypes
import os
import re

import pytest

import fp32_gemm_04_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    names = set()
    for header in HEADERS:
        text = open(header).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:sgemm|sconv2d)_\w+)\s*\(",
                                text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(sg.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(sg.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name


# (M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) with fake but aligned pointers
GOOD = (4, 5, 6, 1.0, 4096, 6, 8192, 5, 0.0, 12288, 5)


def call(**kw):
    names = ("M", "N", "K", "alpha", "A", "lda", "B", "ldb", "beta", "C", "ldc")
    args = dict(zip(names, GOOD))
    args.update(kw)
    return sg.sgemm_f32(*[args[n] for n in names], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3),
    (dict(A=0), -5), (dict(A=4098), -5), (dict(lda=5), -6), (dict(lda=0, K=0, A=0), -6),
    (dict(B=0), -7), (dict(B=8194), -7), (dict(ldb=4), -8),
    (dict(C=0), -10), (dict(C=12290), -10), (dict(ldc=4), -11),
    (dict(M=-1, N=-1), -1), (dict(lda=1, ldb=1), -6),
])
def test_invalid_arguments_are_rejected_first(kw, code):
    assert call(**kw) == code
    assert sg.sgemm_status_string(code).startswith("invalid")


# Calls with valid arguments but fake pointers must never reach a real GPU.
no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU device node is present")


def test_unused_pointers_may_be_null():
    # M == 0 or N == 0: no pointer is needed.
    assert call(M=0, A=0, B=0, C=0) == 0
    assert call(N=0, A=0, B=0, C=0, ldb=1, ldc=1) == 0


@no_gpu
def test_alpha_zero_needs_no_operands():
    # alpha == 0: A and B may be NULL; the checks pass and only the launch
    # (of the C-scaling kernel) fails, because this host has no GPU.
    rc = call(A=0, B=0, alpha=0.0)
    assert rc > 0


def test_quick_return_makes_no_hip_call():
    assert call(M=0) == 0
    assert call(N=0, ldb=1, ldc=1) == 0


@no_gpu
def test_hip_failure_is_a_positive_code():
    rc = call()
    assert rc > 0
    assert "device" in sg.sgemm_status_string(rc).lower()


def test_bad_variant():
    names = ("M", "N", "K", "alpha", "A", "lda", "B", "ldb", "beta", "C", "ldc")
    args = dict(zip(names, GOOD))
    for v in (-1, 4, 15, sg.SGEMM_VARIANT_MFMA_TILE + sg.sgemm_num_mfma_tiles(),
              sg.SGEMM_VARIANT_LADDER - 1, sg.SGEMM_VARIANT_LADDER + sg.SGEMM_LADDER_RUNGS,
              sg.SGEMM_VARIANT_STREAMK_TILE + sg.sgemm_num_mfma_tiles()):
        assert sg.sgemm_f32_variant(v, *[args[n] for n in names], 0) == sg.SGEMM_ERR_BAD_VARIANT
        assert sg.sgemm_plan(v, 4, 5, 6, 6, 5, 5, 1.0, 256)[0] == sg.SGEMM_ERR_BAD_VARIANT


def plan(M, N, K, variant=0, cus=256, alpha=1.0, lda=None, ldb=None, ldc=None):
    rc, text = sg.sgemm_plan(variant, M, N, K, lda or max(1, K), ldb or max(1, N),
                             ldc or max(1, N), alpha, cus)
    assert rc == 0, rc
    return dict(kv.split("=") for kv in text.split()[1:]) | {"kind": text.split()[0]}


def test_plan_quick_paths():
    assert plan(0, 5, 5)["kind"] == "none"
    assert plan(5, 5, 0)["kind"] == "scale"
    assert plan(5, 5, 5, alpha=0.0)["kind"] == "scale"
    assert sg.sgemm_plan(0, 5, 5, 5, 5, 5, 5, 1.0, 0)[0] == -12


def test_plan_covers_every_output_tile():
    for M, N, K in [(5120, 5120, 5120), (384, 14161, 1152), (1, 1, 1), (257, 129, 3)]:
        p = plan(M, N, K)
        bm, bn = int(p["bm"]), int(p["bn"])
        assert int(p["grid"]) == -(-M // bm) * -(-N // bn)


def test_plan_kernel_per_headline_shape():
    for M, N, K in [(5120, 5120, 5120), (1024, 1024, 1024), (384, 14161, 1152),
                    (256, 43264, 1152), (256, 50176, 1024)]:
        assert plan(M, N, K)["kind"] == "mfma"
    assert plan(32, 1605632, 27)["kind"] == "stream16"
    for M, N, K in [(64, 1605632, 147), (64, 559104, 147)]:
        assert plan(M, N, K)["kind"] == "skinny"
    assert plan(5120, 5120, 5120, variant=sg.SGEMM_VARIANT_VALU)["kind"] == "valu"


def test_plan_skinny_details():
    p = plan(64, 1605632, 147)
    assert p["mb"] == "2" and p["kh"] == "74"
    p = plan(32, 1605632, 27)
    assert p["fm"] == "2" and int(p["strips"]) == 1605632 // 64 and int(p["grid"]) == 2 * 256
    assert plan(16, 6400, 5, variant=sg.SGEMM_VARIANT_SKINNY)["fm"] == "1"
    # M <= 32 streams through stream16 only with N % 64 == 0 and aligned rows
    assert plan(32, 1605632 + 4, 27, variant=sg.SGEMM_VARIANT_SKINNY)["kind"] == "skinny"
    assert plan(32, 6400, 27, ldb=6401, variant=sg.SGEMM_VARIANT_SKINNY)["kind"] == "skinny"
    p = plan(32, 1000, 27, variant=sg.SGEMM_VARIANT_SKINNY)
    assert p["mb"] == "1" and p["kh"] == "14"
    # small N stays on the tile kernels unless forced
    assert plan(64, 1000, 27)["kind"] == "mfma"
    assert plan(64, 1000, 27, variant=sg.SGEMM_VARIANT_SKINNY)["kind"] == "skinny"
    rc, _ = sg.sgemm_plan(sg.SGEMM_VARIANT_SKINNY, 65, 10, 10, 10, 10, 10, 1.0, 256)
    assert rc == sg.SGEMM_ERR_VARIANT_SHAPE


def test_plan_vector_paths_follow_leading_dimensions():
    p = plan(384, 14161, 1152)
    assert p["vecA"] == "1" and p["vecB"] == "0"  # N = 14161 is odd
    p = plan(320, 1024, 27)
    assert p["vecA"] == "0" and p["vecB"] == "1"  # K = 27 is odd


def test_plan_fills_the_chip_at_5120():
    # 5120^3 should not leave a partial last round of workgroups.
    p = plan(5120, 5120, 5120)
    assert int(p["grid"]) % 256 == 0


def test_forced_tiles():
    n = sg.sgemm_num_mfma_tiles()
    assert n >= 3
    seen = set()
    for i in range(n):
        p = plan(300, 300, 300, variant=sg.SGEMM_VARIANT_MFMA_TILE + i)
        assert p["kind"] == "mfma"
        seen.add((p["bm"], p["bn"], p["bk"], p["waves"], p["occ"]))
    assert len(seen) == n
    from tests.test_parity import NUM_TILES  # the GPU tests' forced families cover them all
    assert NUM_TILES == n


def test_ladder_rungs():
    """Each rung of the pages' SIMT ladder is its own kernel; the plan names
    it and covers the output with its tile."""
    for r, name in enumerate(sg.LADDER_RUNG_NAMES):
        for M, N, K in [(5120, 5120, 5120), (33, 1605632, 27), (1, 1, 1)]:
            p = plan(M, N, K, variant=sg.SGEMM_VARIANT_LADDER + r)
            assert p["kind"] == "ladder" and p["rung"] == str(r) and p["name"] == name
            tm, tn = (int(x) for x in p["tile"].split("x"))
            assert int(p["grid"]) == -(-M // tm) * -(-N // tn)


def test_ladder_constants_match_header():
    text = open(os.path.join(ROOT, "include", "sgemm.h")).read()
    assert re.search(r"SGEMM_VARIANT_LADDER\s*=\s*%d\b" % sg.SGEMM_VARIANT_LADDER, text)
    assert re.search(r"#define SGEMM_LADDER_RUNGS %d\b" % sg.SGEMM_LADDER_RUNGS, text)
    assert len(sg.LADDER_RUNG_NAMES) == sg.SGEMM_LADDER_RUNGS


def test_streamk_plans():
    """Forced stream-K names its resident workers; the workers never exceed
    the (tile, k-slab) units, and a shape whose tiles fill whole rounds runs
    one tile per workgroup."""
    n = sg.sgemm_num_mfma_tiles()
    for i in range(n):
        for M, N, K in [(300, 200, 1000), (1, 1, 1), (5120, 5120, 5120)]:
            p = plan(M, N, K, variant=sg.SGEMM_VARIANT_STREAMK_TILE + i)
            assert p["kind"] == "mfma" and int(p["streamk"]) > 0
            bm, bn, bk = int(p["bm"]), int(p["bn"]), int(p["bk"])
            units = -(-M // bm) * -(-N // bn) * -(-K // bk)
            assert int(p["streamk"]) <= units
            assert int(p["split"]) < int(p["streamk"])
            # Whole rounds run one tile per workgroup; only the rest is split.
            tiles = -(-M // bm) * -(-N // bn)
            dp, w = int(p["dp"]), int(p["streamk"])
            assert dp % w == 0 and dp <= tiles and tiles - dp < w
            assert int(p["split"]) <= tiles - dp
    assert plan(5120, 5120, 5120)["streamk"] == "0"
    # 576 tiles of 128 over 512 workgroups: one whole round, 64 tiles shared.
    p = plan(3072, 3072, 3072, variant=sg.SGEMM_VARIANT_STREAMK_TILE + 1)
    assert (p["streamk"], p["dp"]) == ("512", "512") and 0 < int(p["split"]) <= 64


def _tune(**kw):
    names = ["M", "N", "K", "alpha", "A", "lda", "B", "ldb", "beta", "C", "ldc"]
    args = dict(M=8, N=8, K=8, alpha=1.0, A=4096, lda=8, B=8192, ldb=8, beta=0.0, C=12288, ldc=8)
    reps = kw.pop("reps", 3)
    args.update(kw)
    return sg.sgemm_tune(*[args[n] for n in names], 0, reps)


def test_tune_checks_arguments_first():
    # Fake pointers: every one of these is rejected before any HIP call.
    assert _tune(M=-1)[0] == -1
    assert _tune(lda=4)[0] == -6
    assert _tune(C=12290)[0] == -10
    assert _tune(reps=0) == (-13, 0, 0.0)
    assert sg.sgemm_status_string(-13).startswith("invalid reps")


def test_tune_quick_return_makes_no_hip_call():
    assert _tune(M=0) == (0, sg.SGEMM_VARIANT_AUTO, 0.0)


def test_tune_reset_and_untuned_plans():
    sg.sgemm_tune_reset()
    for shape in [(5120, 5120, 5120), (64, 1605632, 147), (384, 14161, 1152)]:
        M, N, K = shape
        rc, text = sg.sgemm_plan(0, M, N, K, K, N, N, 1.0, 256)
        assert rc == 0 and "tuned=" not in text


@pytest.mark.parametrize("M,N,K,expect", [
    # one 64 x 64 tile per CU through the four-slab ring
    (1024, 1024, 1024, dict(bm="64", bn="64", waves="2x2", occ="1", load="direct", streamk="0")),
    # one 128 x 128 tile per CU with eight waves
    (2048, 2048, 2048, dict(bm="128", waves="2x4", occ="1", load="direct", streamk="0")),
    # stream-K shares with the eight-wave tile (100 tiles < 256 CUs)
    (1280, 1280, 1280, dict(bm="128", waves="2x4", streamk="256", dp="0")),
    # two whole rounds of 160 x 160
    (5120, 5120, 5120, dict(bm="160", bn="160", occ="2", load="direct", streamk="0")),
    # one whole round plus 64 shared tiles
    (3072, 3072, 3072, dict(bm="128", waves="2x2", streamk="512", dp="512", split="64")),
    # the mid im2col shapes
    (256, 50176, 1024, dict(bm="128", streamk="512", dp="512")),
    (256, 43264, 1152, dict(bm="128", bn="176", waves="4x1", occ="2", load="direct",
                            streamk="0")),
    # odd ldb: B rows at every alignment, the shifted direct-load form; 4 x 64
    # tiles of 96 x 224 fill the CUs once
    (384, 14161, 1152, dict(bm="96", bn="224", waves="2x2", occ="1", load="shifted", vecB="0",
                            streamk="0")),
    (256, 43265, 1152, dict(bm="128", waves="2x2", load="shifted", streamk="0")),
    # the four-slab ring with a K tail, and shifted
    (1000, 1000, 1000, dict(bm="64", occ="1", load="direct", streamk="0")),
    (1000, 1001, 1024, dict(bm="64", occ="1", load="shifted", streamk="0")),
    # K % 16 != 0: no direct-load stream-K
    (384, 14161, 1156, dict(streamk="0")),
    # 4 x 64 tiles of 96 x 224 with B rows aligned too
    (384, 14164, 1152, dict(bm="96", bn="224", load="direct", streamk="0")),
    # 256 tiles of 96 x 96, one per CU, no stream-K
    (1536, 1536, 1536, dict(bm="96", bn="96", streamk="0")),
    # too small for 64 x 64 tiles to fill the CUs: 64 x 32 on all three load paths
    (512, 512, 512, dict(bm="64", bn="32", load="direct")),
    (500, 501, 500, dict(bm="64", bn="32", load="shifted")),
    (333, 517, 259, dict(bm="64", bn="32", load="regs")),
    # where the new tiles lost, the earlier plans stay
    (768, 768, 768, dict(bm="64", bn="64", occ="1")),
    (3328, 3328, 3328, dict(bm="128", bn="128", streamk="512")),
])
def test_selector_choices(M, N, K, expect):
    """The cost model's choices on the configurations, as measured best on
    MI355X (256 CUs); a change to the model that moves them shows here."""
    p = plan(M, N, K)
    for k, v in expect.items():
        assert p[k] == v, (k, p)


def test_valu_tile_choice():
    """The vector-FMA kernel takes the 160 tile where the 128 one leaves a
    part-empty last round of resident workgroups."""
    assert plan(5120, 5120, 5120, variant=sg.SGEMM_VARIANT_VALU)["bm"] == "160"
    assert plan(4096, 4096, 4096, variant=sg.SGEMM_VARIANT_VALU)["bm"] == "128"


def test_k_tail_plans():
    """Direct-load one-tile kernels take any K; the stream-K ones only K a
    multiple of 16, so a forced stream-K variant with a K tail runs the
    register-staged stream-K kernel."""
    assert plan(300, 200, 1000, variant=sg.SGEMM_VARIANT_MFMA_TILE + 1)["load"] == "direct"
    assert plan(300, 200, 1000, variant=sg.SGEMM_VARIANT_STREAMK_TILE + 1)["load"] == "regs"
    assert plan(300, 200, 1008, variant=sg.SGEMM_VARIANT_STREAMK_TILE + 1)["load"] == "direct"
    assert plan(300, 201, 1000, variant=sg.SGEMM_VARIANT_MFMA_TILE + 1)["load"] == "shifted"
    assert plan(300, 200, 7, variant=sg.SGEMM_VARIANT_MFMA_TILE + 6, lda=8)["load"] == "direct"
    # A rows not 16-byte aligned: no direct load
    assert plan(300, 200, 1000, variant=sg.SGEMM_VARIANT_MFMA_TILE + 1, lda=1001)["load"] == "regs"
