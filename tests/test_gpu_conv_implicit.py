"""GPU parity of the general INT8 convolution qconv2d_s8 (implicit GEMM,
1x1 fastway and the explicit-im2col route, all with dilation) against the
oracle's direct convolution (O4) and requantization (O3): bit-exact for every
int8 and int32 output.  Weights with zero points are checked against the
im2col reference (O4b) followed by the affine GEMM (O1)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import conv_qpack_weights_amd as qp
    return qp


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    return t.cpu().numpy()


def _first_diff(got, want, what, acc=None):
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        extra = "" if acc is None else " (oracle int32 acc %d)" % acc[i]
        raise AssertionError("%s: %d mismatches, first at %s: gpu=%s oracle=%s%s"
                             % (what, len(bad), i, got[i], want[i], extra))


def _case(qp, orc, X, zp_in, s_in, Wt, s_w, bias, stride, pad, dil, s_out, zp_out, relu):
    OC, _, KH, KW = Wt.shape
    print("conv case", X.shape, Wt.shape, stride, pad, dil, flush=True)
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(s_w))
    mab = int(np.abs(bias).max()) if bias is not None else 0
    dX = _dev(X)
    dbias = None if bias is None else _dev(bias)
    y32 = _host(qp.qconv2d_s8(dX, s_in, zp_in, blob, info, KH, KW, stride, pad, dil, dbias, mab,
                              out_dtype="s32"))
    y8 = _host(qp.qconv2d_s8(dX, s_in, zp_in, blob, info, KH, KW, stride, pad, dil, dbias, mab,
                             s_out, zp_out, relu))
    acc = orc.conv2d_direct(X, zp_in, Wt, stride, pad, bias, dil)
    want8, _ = orc.requant_matrix(acc.reshape(-1, OC), s_in, s_w, s_out, zp_out, relu)
    _first_diff(y32, acc.astype(np.int32), "conv int32")
    _first_diff(y8.reshape(-1, OC), want8, "conv int8", acc.reshape(-1, OC))
    return y8


def test_conv3x3_workload_implicit(qp, orc):
    c = synth.conv3x3_nhwc()
    y8 = _case(qp, orc, c["X"], c["zp_in"], c["s_in"], c["W"], c["s_w"], c["bias"], c["stride"],
               c["pad"], (1, 1), c["s_out"], c["zp_out"], c["relu"])
    # the explicit route gives the same bytes
    blob, info = qp.pack_s8(_dev(c["W"]), scales=_dev(c["s_w"]))
    ex = _host(qp.qconv2d_s8_im2col(_dev(c["X"]), c["s_in"], c["zp_in"], blob, info, 3, 3,
                                    c["stride"], c["pad"], _dev(c["bias"]), 1000, c["s_out"],
                                    c["zp_out"], c["relu"]))
    assert np.array_equal(ex, y8)


@pytest.mark.parametrize("geom", [
    # implicit route (C % 16 == 0): strides, asymmetric pads, dilations,
    # batches, ragged pixel and channel counts, narrow and wide channel tiles
    dict(NB=2, H=9, W=11, C=16, OC=20, KH=3, KW=3, stride=(1, 1), pad=(1, 1, 1, 1), dil=(1, 1)),
    dict(NB=1, H=13, W=10, C=32, OC=70, KH=3, KW=2, stride=(2, 1), pad=(0, 1, 2, 0), dil=(1, 1)),
    dict(NB=3, H=12, W=12, C=48, OC=33, KH=3, KW=3, stride=(1, 1), pad=(2, 2, 2, 2), dil=(2, 2)),
    dict(NB=1, H=17, W=15, C=16, OC=8, KH=3, KW=3, stride=(2, 2), pad=(3, 1, 0, 2), dil=(3, 1)),
    dict(NB=2, H=8, W=8, C=64, OC=64, KH=5, KW=5, stride=(1, 1), pad=(2, 2, 2, 2), dil=(1, 1)),
    dict(NB=1, H=7, W=7, C=80, OC=96, KH=7, KW=7, stride=(1, 1), pad=(3, 3, 3, 3), dil=(1, 1)),
    dict(NB=1, H=5, W=6, C=16, OC=5, KH=1, KW=1, stride=(2, 2), pad=(1, 0, 1, 0), dil=(1, 1)),
    # K = 32832, just under the int32 bound K*65025 < 2^31 (513 K-steps);
    # and pads and dilations much larger than the image
    dict(NB=1, H=3, W=4, C=3648, OC=16, KH=3, KW=3, stride=(1, 1), pad=(1, 1, 1, 1), dil=(1, 1)),
    dict(NB=1, H=4, W=3, C=16, OC=8, KH=2, KW=2, stride=(1, 1), pad=(40, 30, 0, 0), dil=(20, 15)),
    # 1x1 fastway (the GEMM on x itself), K a multiple of 64 and not
    dict(NB=2, H=7, W=9, C=64, OC=40, KH=1, KW=1, stride=(1, 1), pad=(0, 0, 0, 0), dil=(1, 1)),
    dict(NB=1, H=6, W=5, C=24, OC=17, KH=1, KW=1, stride=(1, 1), pad=(0, 0, 0, 0), dil=(2, 3)),
    # explicit route (C % 16 != 0), with dilation
    dict(NB=2, H=10, W=9, C=3, OC=12, KH=3, KW=3, stride=(1, 2), pad=(2, 1, 2, 1), dil=(2, 1)),
    dict(NB=1, H=8, W=8, C=24, OC=9, KH=2, KW=3, stride=(1, 1), pad=(0, 0, 1, 1), dil=(1, 2)),
])
def test_conv_general_geometry(qp, orc, geom):
    rng = np.random.default_rng(geom["C"] * 7 + geom["OC"])
    X = rng.integers(-128, 128, (geom["NB"], geom["H"], geom["W"], geom["C"])).astype(np.int8)
    Wt = rng.integers(-127, 128, (geom["OC"], geom["C"], geom["KH"], geom["KW"])).astype(np.int8)
    s_w = rng.uniform(0.001, 0.01, geom["OC"]).astype(np.float32)
    bias = rng.integers(-1000, 1001, geom["OC"]).astype(np.int32)
    _case(qp, orc, X, int(rng.integers(-128, 128)), 0.05, Wt, s_w, bias, geom["stride"],
          geom["pad"], geom["dil"], 0.1, int(rng.integers(-10, 10)), bool(geom["C"] % 32 == 0))


@pytest.mark.parametrize("seed", range(6))
def test_conv_random_geometry_implicit(qp, orc, seed):
    rng = np.random.default_rng(900 + seed)
    NB, H, W = int(rng.integers(1, 4)), int(rng.integers(4, 20)), int(rng.integers(4, 20))
    C, OC = 16 * int(rng.integers(1, 6)), int(rng.integers(1, 100))
    KH, KW = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    stride = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    pad = tuple(int(rng.integers(0, d * (k - 1) + 1)) for k, d in ((KH, dil[0]), (KW, dil[1]),
                                                                  (KH, dil[0]), (KW, dil[1])))
    if H + pad[0] + pad[2] < dil[0] * (KH - 1) + 1 or W + pad[1] + pad[3] < dil[1] * (KW - 1) + 1:
        pytest.skip("kernel larger than the padded input")
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-127, 128, (OC, C, KH, KW)).astype(np.int8)
    s_w = rng.uniform(0.001, 0.01, OC).astype(np.float32)
    bias = rng.integers(-1000, 1001, OC).astype(np.int32) if seed % 3 else None
    _case(qp, orc, X, int(rng.integers(-128, 128)), 0.05, Wt, s_w, bias, stride, pad, dil, 0.1,
          int(rng.integers(-10, 10)), bool(seed % 2))


@pytest.mark.parametrize("C,KH,pad", [(32, 3, (1, 1, 1, 1)), (5, 3, (1, 1, 1, 1)),
                                      (48, 1, (0, 0, 0, 0))])
def test_conv_weight_zero_points(qp, orc, C, KH, pad):
    """Per-channel weight zero points (the row-sum correction): implicit,
    explicit and fastway routes against im2col (O4b) + the affine GEMM (O1)."""
    rng = np.random.default_rng(77 + C)
    NB, H, W, OC = 2, 9, 10, 37
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-128, 128, (OC, C, KH, KH)).astype(np.int8)
    zw = rng.integers(-20, 21, OC).astype(np.int32)
    s_w = rng.uniform(0.001, 0.01, OC).astype(np.float32)
    bias = rng.integers(-1000, 1001, OC).astype(np.int32)
    zp_in, s_in, s_out, zp_out = -9, 0.05, 0.2, 4
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(s_w), zero_points=_dev(zw))
    dX = _dev(X)
    y32 = _host(qp.qconv2d_s8(dX, s_in, zp_in, blob, info, KH, KH, (1, 1), pad, (1, 1),
                              _dev(bias), 1000, out_dtype="s32"))
    y8 = _host(qp.qconv2d_s8(dX, s_in, zp_in, blob, info, KH, KH, (1, 1), pad, (1, 1),
                             _dev(bias), 1000, s_out, zp_out, False))
    col = orc.im2col(X, zp_in, KH, KH, (1, 1), pad)
    Bnk = Wt.transpose(0, 2, 3, 1).reshape(OC, -1)
    acc = orc.gemm_affine(col, zp_in, Bnk, zw, bias, b_is_nk=True)
    want8, _ = orc.requant_matrix(acc, s_in, s_w, s_out, zp_out, False)
    _first_diff(y32.reshape(-1, OC), acc.astype(np.int32), "zp conv int32")
    _first_diff(y8.reshape(-1, OC), want8, "zp conv int8", acc)


def test_conv_wide_batch_config(qp, orc):
    """Enough pixels for the 128-pixel tile configuration: NB=64 32x32x16 ->
    128 channels, 3x3, pad 1; every int32 and int8 output against O4 and O3
    (the oracle runs the images on host threads)."""
    rng = np.random.default_rng(4242)
    NB, H, W, C, OC = 64, 32, 32, 16, 128
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-127, 128, (OC, C, 3, 3)).astype(np.int8)
    s_w = rng.uniform(0.001, 0.01, OC).astype(np.float32)
    bias = rng.integers(-1000, 1001, OC).astype(np.int32)
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(s_w))
    dX = _dev(X)
    y32 = _host(qp.qconv2d_s8(dX, 0.05, 3, blob, info, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1),
                              _dev(bias), 1000, out_dtype="s32"))
    acc = orc.rows_in_threads(orc.conv2d_direct, X, 3, Wt, (1, 1), (1, 1, 1, 1), bias)
    _first_diff(y32, acc.astype(np.int32), "wide conv int32")
    y8 = _host(qp.qconv2d_s8(dX, 0.05, 3, blob, info, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1),
                             _dev(bias), 1000, 0.1, 0, True))
    want8, _ = orc.requant_matrix(acc.reshape(-1, OC), 0.05, s_w, 0.1, 0, True)
    _first_diff(y8.reshape(-1, OC), want8, "wide conv int8")


def test_conv_rejects_bad_dilation(qp):
    import torch
    Wt = np.ones((4, 16, 3, 3), np.int8)
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(np.full(4, 0.01, np.float32)))
    X = torch.zeros((1, 4, 4, 16), dtype=torch.int8, device="cuda")
    for dil in [(0, 1), (1, -1)]:
        with pytest.raises(Exception):
            qp.qconv2d_s8(X, 0.05, 0, blob, info, 3, 3, (1, 1), (1, 1, 1, 1), dil)
    with pytest.raises(Exception):   # dilated span 5 > padded 4 rows
        qp.qconv2d_s8(X, 0.05, 0, blob, info, 3, 3, (1, 1), (0, 0, 0, 0), (2, 2))
