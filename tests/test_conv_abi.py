"""Host logic of the convolution entry points, on a host without a GPU:
argument checks come before any HIP call, quick returns make none, and the
plan picks the stem kernel for the geometries it is built for, the matrix-core
tile kernel where its tiles keep the CUs busier, and the general kernel
otherwise."""
import os

import pytest

import fp32_gemm_04_amd as sg

# (batch, C, H, W, M, R, S, sh, sw, ph, pw) of the 7x7 stem reading, and
# fake aligned pointers for X, Wt, Y
GEOM = dict(batch=2, channels=3, height=224, width=224, out_channels=64, kernel_h=7, kernel_w=7,
            stride_h=2, stride_w=2, pad_h=3, pad_w=3)
NAMES = list(GEOM)


def call(**kw):
    g = dict(GEOM)
    g.update({k: v for k, v in kw.items() if k in GEOM})
    K = g["channels"] * g["kernel_h"] * g["kernel_w"]
    oh = (g["height"] + 2 * g["pad_h"] - g["kernel_h"]) // max(g["stride_h"], 1) + 1
    ow = (g["width"] + 2 * g["pad_w"] - g["kernel_w"]) // max(g["stride_w"], 1) + 1
    args = dict(alpha=1.0, X=4096, Wt=8192, ldw=K, beta=0.0, Y=12288,
                ldy=max(1, g["batch"] * oh * ow))
    args.update({k: v for k, v in kw.items() if k not in GEOM})
    return sg.sconv2d_f32(*[g[n] for n in NAMES], args["alpha"], args["X"], args["Wt"],
                          args["ldw"], args["beta"], args["Y"], args["ldy"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -1), (dict(channels=0), -2), (dict(height=0), -3), (dict(width=0), -4),
    (dict(out_channels=-1), -5), (dict(kernel_h=0), -6), (dict(kernel_w=0), -7),
    (dict(stride_h=0), -8), (dict(stride_w=0), -9), (dict(pad_h=-1), -10), (dict(pad_w=-1), -11),
    (dict(pad_h=2 ** 30), -10), (dict(pad_w=2 ** 30), -11),
    (dict(kernel_h=231), -6), (dict(kernel_w=231), -7),
    (dict(X=0), -13), (dict(X=4098), -13), (dict(Wt=0), -14), (dict(ldw=146), -15),
    (dict(Y=0), -17), (dict(Y=12290), -17), (dict(ldy=1000), -18),
])
def test_invalid_arguments(kw, code):
    assert call(**kw) == code


def test_quick_returns_need_no_pointers():
    assert call(batch=0, X=0, Wt=0, Y=0, ldy=1) == 0
    assert call(out_channels=0, X=0, Wt=0, Y=0) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU device node is present")
def test_alpha_zero_reads_no_operands():
    assert call(alpha=0.0, X=0, Wt=0) > 0  # the checks pass; the launch fails without a GPU


def test_bad_variant_first():
    for v in (-1, 6, 100):
        rc = sg.sconv2d_f32_variant(v, *[GEOM[n] for n in NAMES], 1.0, 0, 0, 0, 0.0, 0, 0, 0)
        assert rc == sg.SGEMM_ERR_BAD_VARIANT


def plan(variant=0, cus=256, **kw):
    g = dict(GEOM)
    g.update(kw)
    rc, text = sg.sconv2d_plan(variant, *[g[n] for n in NAMES], cus)
    assert rc == 0, rc
    return text


def test_plans():
    assert sg.sconv2d_num_stem_kernels() >= 2
    p = plan(batch=128)
    assert p.startswith("stem mb=2 k=147") and "strips=6272" in p and "grid=512" in p, p
    p = plan(batch=128, out_channels=32, kernel_h=3, kernel_w=3, pad_h=1, pad_w=1)
    assert p.startswith("stem mb=1 k=27") and "grid=768" in p, p  # three per CU
    assert plan(out_channels=20).startswith("stem mb=1")
    assert plan(variant=sg.SCONV_VARIANT_GENERAL).startswith("general")
    # outside the stem kernels' geometries: general, and the forced stem form refuses
    for kw in [dict(channels=4), dict(stride_h=1), dict(out_channels=65), dict(width=256),
               dict(width=64), dict(pad_w=5), dict(kernel_h=5)]:
        assert plan(**kw).startswith("general"), kw
        g = dict(GEOM)
        g.update(kw)
        rc, _ = sg.sconv2d_plan(sg.SCONV_VARIANT_STEM, *[g[n] for n in NAMES], 256)
        assert rc == sg.SGEMM_ERR_VARIANT_SHAPE, kw
    # the mid-size readings: 3x3 stride 1 pad 1 over 128 channels, batch 1.
    # 384 x 14161: 2 x 111 tiles of 192 x 128 fill 256 CUs once, where
    # 3 x 111 of 128 x 128 would put two on some CUs; 256 x 43264: 128 x 128.
    mid = dict(batch=1, channels=128, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1, pad_h=1,
               pad_w=1)
    p = plan(height=119, width=119, out_channels=384, **mid)
    assert p == "tap bm=192 bn=128 waves=8 k=1152 grid=222 oh=119 ow=119", p
    p = plan(height=208, width=208, out_channels=256, **mid)
    assert p == "tap bm=128 bn=128 waves=4 k=1152 grid=676 oh=208 ow=208", p
    p = plan(variant=sg.SCONV_VARIANT_DIRECT, height=208, width=208, out_channels=256, **mid)
    assert p == "direct bm=128 bn=128 waves=4 k=1152 grid=676 oh=208 ow=208", p
    # the tap form: 3x3 filters over a multiple of 4 channels
    assert plan(variant=sg.SCONV_VARIANT_TAP, height=20, width=20, out_channels=64,
                **mid).startswith("tap")
    for kw in [dict(channels=6), dict(kernel_h=1, kernel_w=1)]:
        g = dict(GEOM, height=20, width=20, out_channels=64)
        g.update(mid)
        g.update(kw)
        rc, _ = sg.sconv2d_plan(sg.SCONV_VARIANT_TAP, *[g[n] for n in NAMES], 256)
        assert rc == sg.SGEMM_ERR_VARIANT_SHAPE, kw
    p = plan(variant=sg.SCONV_VARIANT_TILE, height=208, width=208, out_channels=256, **mid)
    assert p == "tile bm=128 bn=128 waves=4 k=1152 grid=676 oh=208 ow=208", p
    # the direct form: 3x3 and 1x1 filters with K % 16 == 0 only
    assert plan(variant=sg.SCONV_VARIANT_DIRECT, height=20, width=20, out_channels=64,
                **mid).startswith("direct")
    for kw in [dict(channels=5), dict(kernel_h=5, kernel_w=5)]:
        g = dict(GEOM, height=20, width=20, out_channels=64)
        g.update(mid)
        g.update(kw)
        rc, _ = sg.sconv2d_plan(sg.SCONV_VARIANT_DIRECT, *[g[n] for n in NAMES], 256)
        assert rc == sg.SGEMM_ERR_VARIANT_SHAPE, kw
    assert plan(variant=sg.SCONV_VARIANT_GENERAL, height=208, width=208, out_channels=256,
                **mid).startswith("general tile=64x64")
    # a small problem keeps the general kernel's finer tiles; the forced
    # tile form still takes it; 1x1 filters have tile kernels too
    small = dict(batch=2, channels=16, height=17, width=19, out_channels=33, kernel_h=3,
                 kernel_w=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1)
    assert plan(**small).startswith("general")
    assert plan(variant=sg.SCONV_VARIANT_TILE, **small).startswith("tile bm=64 bn=128")
    # a pointwise layer (1x1, stride 1, no padding) runs as one product per image
    pw = dict(batch=8, channels=256, height=56, width=56, out_channels=512, kernel_h=1,
              kernel_w=1, stride_h=1, stride_w=1, pad_h=0, pad_w=0)
    assert plan(**pw) == "gemm images=8 m=512 n=3136 k=256 oh=56 ow=56", plan(**pw)
    p = plan(variant=sg.SCONV_VARIANT_DIRECT, **pw)
    assert p.startswith("direct") and "k=256" in p, p
    p = plan(variant=sg.SCONV_VARIANT_TILE, **dict(pw, channels=250))
    assert p.startswith("tile") and "k=250" in p, p
    # with a stride or padding, a 1x1 filter takes the implicit forms
    p = plan(**dict(pw, stride_h=2, stride_w=2))
    assert p.startswith("direct") and "k=256" in p, p
    p = plan(**dict(pw, channels=250, pad_h=1, pad_w=1))
    assert p.startswith("tile") and "k=250" in p, p
    # the tile kernels take any filter; they refuse inputs of 2^31 bytes or more
    for kw in [dict(), dict(kernel_h=3), dict(kernel_h=5, kernel_w=5)]:
        assert plan(variant=sg.SCONV_VARIANT_TILE, **kw).startswith("tile"), kw
    g = dict(GEOM, batch=4096)  # 4096 * 3 * 224 * 224 * 4 bytes > 2^31
    rc, _ = sg.sconv2d_plan(sg.SCONV_VARIANT_TILE, *[g[n] for n in NAMES], 256)
    assert rc == sg.SGEMM_ERR_VARIANT_SHAPE
    assert plan(batch=4096).startswith("general")  # Y over 2^32 bytes: not the stem either
    assert plan(out_channels=0) == "none"


def test_im2col_arguments():
    args = [2, 3, 224, 224, 7, 7, 2, 2, 3, 3, 4096, 8192, 2 * 112 * 112]
    if not os.path.exists("/dev/kfd"):  # fake pointers: launch only where there is no GPU
        assert sg.sgemm_im2col_f32(*args, 0) > 0
    for i, code in [(0, -1), (1, -2), (2, -3), (3, -4), (4, -5), (5, -6), (6, -7), (7, -8)]:
        bad = list(args)
        bad[i] = 0 if i < 8 else bad[i]
        if i == 0:
            bad[0] = -1
        assert sg.sgemm_im2col_f32(*bad, 0) == code, (i, code)
    bad = list(args)
    bad[8] = -1
    assert sg.sgemm_im2col_f32(*bad, 0) == -9
    bad = list(args)
    bad[10] = 0
    assert sg.sgemm_im2col_f32(*bad, 0) == -11
    bad = list(args)
    bad[11] = 8194
    assert sg.sgemm_im2col_f32(*bad, 0) == -12
    bad = list(args)
    bad[12] = 100
    assert sg.sgemm_im2col_f32(*bad, 0) == -13
    assert sg.sgemm_im2col_f32(0, 3, 224, 224, 7, 7, 2, 2, 3, 3, 0, 0, 1, 0) == 0
