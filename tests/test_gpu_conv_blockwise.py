"""GPU parity of the channel-blocked int8 convolution with f32 output
(qconv2d_s8_blockwise_f32: one weight scale per output channel and block of
input channels) against oracle O4c: |gpu - oracle| <= 1e-5 * max(1, |oracle|)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
RTOL = 1e-5


@pytest.fixture(scope="module")
def qp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import conv_qpack_weights_amd as qp
    return qp


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check_close(got, want, what):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = RTOL * np.maximum(1.0, np.abs(want.astype(np.float64)))
    bad = np.argwhere(err > tol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d outside 1e-5*max(1,|o|); first at %s gpu=%r oracle=%r"
                             % (what, len(bad), i, float(got[i]), float(want[i])))


def _case(qp, orc, NB, H, W, C, OC, KH, KW, icb, stride, pad, dil, seed, lo=-np.inf, hi=np.inf):
    print("blockwise conv", NB, H, W, C, OC, KH, KW, icb, stride, pad, dil, flush=True)
    rng = np.random.default_rng(seed)
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-127, 128, (OC, C, KH, KW)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (OC, C // icb)).astype(np.float32)
    bias = rng.uniform(-1, 1, OC).astype(np.float32)
    zx, sx = int(rng.integers(-20, 21)), 0.05
    blob, info = qp.pack_s8_blockwise(_dev(Wt), _dev(sw), block=icb)
    y = qp.qconv2d_s8_blockwise_f32(_dev(X), sx, zx, blob, info, KH, KW, stride, pad, dil,
                                    _dev(bias), lo, hi).cpu().numpy()
    want = orc.rows_in_threads(orc.conv2d_blockwise_f32, X, zx, sx, Wt, icb, sw, stride, pad,
                               bias, dil, lo, hi)
    assert y.shape == want.shape
    _check_close(y, want, "blockwise conv")
    return blob, info, sw


def test_blockwise_conv_56x56x64(qp, orc):
    _case(qp, orc, 1, 56, 56, 64, 64, 3, 3, 64, (1, 1), (1, 1, 1, 1), (1, 1), 1, 0.0, 6.0)


@pytest.mark.parametrize("g", [
    dict(NB=2, H=14, W=13, C=128, OC=70, KH=3, KW=3, icb=64, stride=(1, 1), pad=(1, 1, 1, 1),
         dil=(1, 1)),
    dict(NB=1, H=12, W=12, C=128, OC=48, KH=3, KW=3, icb=128, stride=(2, 2), pad=(2, 1, 0, 2),
         dil=(2, 1)),
    dict(NB=3, H=9, W=9, C=256, OC=33, KH=1, KW=1, icb=128, stride=(1, 1), pad=(0, 0, 0, 0),
         dil=(1, 1)),
    dict(NB=1, H=10, W=11, C=64, OC=16, KH=5, KW=5, icb=64, stride=(1, 1), pad=(2, 2, 2, 2),
         dil=(1, 1)),
    dict(NB=2, H=7, W=8, C=192, OC=96, KH=2, KW=3, icb=64, stride=(1, 2), pad=(0, 1, 1, 0),
         dil=(1, 1)),
])
def test_blockwise_conv_geometry(qp, orc, g):
    _case(qp, orc, g["NB"], g["H"], g["W"], g["C"], g["OC"], g["KH"], g["KW"], g["icb"],
          g["stride"], g["pad"], g["dil"], g["C"] + g["OC"])


def test_blockwise_conv_deep_k(qp, orc):
    """K = 18432 (2048 channels, 3x3): a 32-channel tile's scales (288
    blocks) exceed the workgroup's 32 KiB LDS copy and are read from memory
    every step; K = 16384 (1024 channels, 4x4) fills that copy exactly.  The
    running sum over 256-288 blocks is what the plain 1e-5 bound checks."""
    _case(qp, orc, 1, 4, 5, 2048, 40, 3, 3, 64, (1, 1), (1, 1, 1, 1), (1, 1), 9)
    _case(qp, orc, 1, 5, 5, 1024, 32, 4, 4, 64, (1, 1), (2, 1, 1, 2), (1, 1), 10, -3.0, 3.0)
    # the same depth with enough pixels for one tile per wave (no K split)
    _case(qp, orc, 32, 16, 16, 1024, 64, 3, 3, 64, (1, 1), (1, 1, 1, 1), (1, 1), 11)


def test_blockwise_conv_wide_batch(qp, orc):
    """Enough pixels for the 32-pixel-per-wave configuration (128 x 16x16
    images); every image against the oracle (run on host threads)."""
    import torch
    rng = np.random.default_rng(77)
    NB, H, W, C, OC = 128, 16, 16, 64, 64
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-127, 128, (OC, C, 3, 3)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (OC, 1)).astype(np.float32)
    blob, info = qp.pack_s8_blockwise(_dev(Wt), _dev(sw), block=64)
    y = qp.qconv2d_s8_blockwise_f32(_dev(X), 0.05, 3, blob, info, 3, 3, (1, 1),
                                    (1, 1, 1, 1)).cpu().numpy()
    want = orc.rows_in_threads(orc.conv2d_blockwise_f32, X, 3, 0.05, Wt, 64, sw, (1, 1),
                               (1, 1, 1, 1))
    _check_close(y, want, "wide blockwise conv")


def test_blockwise_conv_scales_repeat_over_taps(qp, orc):
    blob, info, sw = _case(qp, orc, 1, 6, 6, 128, 8, 3, 3, 64, (1, 1), (1, 1, 1, 1), (1, 1), 5)
    _, sc, _, _ = qp.qunpack_weights(blob, info, values=False)
    sc = sc.cpu().numpy()
    assert sc.shape == (8, 18)                      # 9 taps x 2 channel blocks
    assert np.array_equal(sc, np.tile(sw, (1, 9)))


def test_blockwise_conv_rejects_unsupported(qp):
    import torch
    Wt = torch.zeros((8, 96, 3, 3), dtype=torch.int8, device="cuda")
    with pytest.raises(qp.QPackError):        # 64 does not divide 96
        qp.pack_s8_blockwise(Wt, torch.ones((8, 1), device="cuda"), block=64)
    Wt = torch.zeros((8, 8, 1, 1), dtype=torch.int8, device="cuda")
    with pytest.raises(qp.QPackError):        # 64 does not divide IC = 8
        qp.pack_s8_blockwise(Wt, torch.ones((8, 1), device="cuda"), block=64)
