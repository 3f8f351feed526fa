"""GPU parity of the block-quantized int8 weight path (qgemm_a8w8_blockwise_*:
dynamically quantized int8 activations, int8 weights with one f32 scale per
channel and block of 64 or 128 K, f32 out with bias and clamp) against the
oracle (O5 then O6 with int8 weights and the block as the group):
|gpu - oracle| <= 1e-5 * max(1, |oracle|)."""
import numpy as np
import pytest

import synth

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


def _host(t):
    return t.cpu().numpy()


def _check_close(got, want, what):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = RTOL * np.maximum(1.0, np.abs(want.astype(np.float64)))
    bad = np.argwhere(err > tol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d outside 1e-5*max(1,|o|); first at %s gpu=%r oracle=%r"
                             % (what, len(bad), i, float(got[i]), float(want[i])))


def _inputs(M, N, K, bs, seed):
    rng = np.random.default_rng(seed)
    d = synth.a8w4(synth.BASE_SEED + seed, M, N, K)     # X N(0,1), bias U[-1,1]
    W = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (N, (K + bs - 1) // bs)).astype(np.float32)
    return d["X"], W, sw, d["bias"]


def _case(qp, orc, M, N, K, bs, seed, rows=None, prequant=False, lo=-6.0, hi=6.0):
    print("a8w8b case", M, N, K, bs, prequant, flush=True)
    X, W, sw, bias = _inputs(M, N, K, bs, seed)
    blob, info = qp.pack_s8_blockwise(_dev(W), _dev(sw), block=bs)
    assert info.format == 5 and info.group == bs
    if prequant:
        import torch
        q = torch.zeros((M, info.Kpad), dtype=torch.int8, device="cuda")
        q, s, z = qp.qquantize_rows_s8(_dev(X), q=q)
        Y = _host(qp.qgemm_a8w8_blockwise_prequant_f32(q, s, z, blob, info, _dev(bias), lo, hi))
    else:
        Y = _host(qp.qgemm_a8w8_blockwise_f32(_dev(X), blob, info, _dev(bias), lo, hi))
    Xs = X if rows is None else X[rows]
    want = orc.rows_in_threads(orc.a8w4_forward, Xs, W, sw, bias, lo, hi, group=bs)
    _check_close(Y if rows is None else Y[rows], want, "a8w8 blockwise output")
    return blob, info, W, sw


@pytest.mark.parametrize("bs", [64, 128])
def test_a8w8b_gemv_4096(qp, orc, bs):
    _case(qp, orc, 1, 4096, 4096, bs, 1)


@pytest.mark.parametrize("M,bs", [(16, 128), (16, 64), (128, 128), (128, 64)])
def test_a8w8b_gemm_11008x4096(qp, orc, M, bs):
    _case(qp, orc, M, 11008, 4096, bs, 2 + M)


@pytest.mark.parametrize("M,N,K,bs,prequant", [(1, 70, 96, 64, False), (2, 130, 200, 128, True),
                                               (5, 77, 1000, 64, False), (17, 100, 256, 128, False),
                                               (33, 48, 160, 64, True), (40, 33, 67, 128, False),
                                               (130, 48, 320, 64, False)])
def test_a8w8b_shapes_and_tails(qp, orc, M, N, K, bs, prequant):
    _case(qp, orc, M, N, K, bs, M + N + K, prequant=prequant)


@pytest.mark.parametrize("N,K,bs", [(33, 1000, 128), (48, 20000, 64), (16, 32768, 128),
                                    (17, 32769, 64), (40, 4096, 64), (1, 64, 64), (3, 1, 128)])
def test_a8w8b_gemv_fused_shapes(qp, orc, N, K, bs):
    """One row from f32: the fused GEMV (the row quantized inside every
    workgroup, no workspace) for Kpad <= 32768, the two launches beyond;
    ragged N and K, several batches of K steps per wave."""
    _case(qp, orc, 1, N, K, bs, N + K)
    Kpad = (K + 127) // 128 * 128
    info = qp.pack_s8_blockwise(_dev(np.zeros((N, K), np.int8)),
                                _dev(np.ones((N, (K + bs - 1) // bs), np.float32)), block=bs)[1]
    assert (qp.qgemm_a8w8_blockwise_f32_ws_size(1, info) == 0) == (Kpad <= 32768)


def test_a8w8b_gemv_fused_unaligned_row(qp, orc):
    """A row that starts 4 bytes past a 16-byte boundary takes the
    quantizer's scalar loads."""
    import torch
    X, W, sw, bias = _inputs(1, 70, 900, 64, 77)
    blob, info = qp.pack_s8_blockwise(_dev(W), _dev(sw), block=64)
    big = torch.zeros((1, 904), dtype=torch.float32, device="cuda")
    big[:, 1:901] = _dev(X)
    Xv = big[:, 1:901]
    assert Xv.data_ptr() % 16 == 4
    Y = _host(qp.qgemm_a8w8_blockwise_f32(Xv, blob, info, _dev(bias), -6.0, 6.0))
    want = orc.a8w4_forward(X, W, sw, bias, -6.0, 6.0, group=64)
    _check_close(Y, want, "fused a8w8 GEMV, unaligned row")


def test_a8w8b_unpack_and_conv_weights(qp, orc):
    """A 1x1 convolution's OIHW weights pack as K = C; unpack returns the
    values, the block scales and the dequantized weights (O9)."""
    rng = np.random.default_rng(9)
    Wt = rng.integers(-128, 128, (24, 256, 1, 1)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (24, 4)).astype(np.float32)
    blob, info = qp.pack_s8_blockwise(_dev(Wt), _dev(sw), block=64)
    w, sc, zp, dq = qp.qunpack_weights(blob, info, dequant=True)
    W = Wt.reshape(24, 256)
    assert zp is None
    assert np.array_equal(_host(w), W) and np.array_equal(_host(sc), sw)
    assert np.array_equal(_host(dq), orc.dequant_weights_s4(W, sw, 64))


def test_a8w8b_rejects_unsupported(qp):
    import torch
    W = torch.zeros((16, 128), dtype=torch.int8, device="cuda")
    with pytest.raises(qp.QPackError):      # block of 32: not a whole MFMA K-step
        qp.pack_s8_blockwise(W, torch.ones((16, 4), device="cuda"), block=32)
    blob, info = qp.pack_s4(W, torch.ones((16, 4), device="cuda"))
    with pytest.raises(qp.QPackError):      # an int4 blob is not a block-quantized int8 blob
        qp.qgemm_a8w8_blockwise_f32(torch.zeros((1, 128), device="cuda"), blob, info)
