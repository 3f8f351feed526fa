"""Run-to-run and launch-geometry agreement.  Every kernel reduces in a
fixed order (no atomics), so repeated calls are bitwise equal, including the
f32 paths whose waves split K and add their partial sums through LDS.
Integer results do not depend on the tile configuration a shape selects:
rows of a large GEMM equal the same rows computed as a small one."""
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


def _repeat_equal(call, n=10):
    first = call().cpu().numpy()
    for i in range(n):
        assert np.array_equal(call().cpu().numpy(), first), "call %d differs" % i
    return first


def test_int8_gemm_rows_independent_of_tile_configuration(qp):
    """M = 4096, N = 4096 takes the 256x256 tiles; its first 64 and last 40
    rows alone take the 64x64 tiles: the int8 and int32 outputs agree."""
    print("geometry: int8 GEMM 4096x4096x256 vs row slices", flush=True)
    rng = np.random.default_rng(61)
    M, N, K = 4096, 4096, 256
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    W = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s_w = rng.uniform(0.001, 0.01, N).astype(np.float32)
    bias = rng.integers(-1000, 1001, N).astype(np.int32)
    blob, info = qp.pack_s8(_dev(W), scales=_dev(s_w))
    dA, db = _dev(A), _dev(bias)
    for out_dtype in ("s8", "s32"):
        full = qp.qgemm_s8s8_requant(dA, 0.01, 5, blob, info, db, 1000, 0.5, -3, True,
                                     out_dtype=out_dtype).cpu().numpy()
        for lo, hi in ((0, 64), (M - 40, M)):
            part = qp.qgemm_s8s8_requant(dA[lo:hi].contiguous(), 0.01, 5, blob, info, db, 1000,
                                         0.5, -3, True, out_dtype=out_dtype).cpu().numpy()
            assert np.array_equal(part, full[lo:hi]), (out_dtype, lo, hi)


@pytest.mark.parametrize("M", [16, 128])
def test_a8w4_gemm_repeats_bitwise(qp, M):
    print("determinism: A8W4 GEMM M=%d" % M, flush=True)
    a = synth.a8w4(synth.BASE_SEED + 51, M, 1024, 4096)
    blob, info = qp.pack_s4(_dev(a["W"]), _dev(a["sw"]))
    X, b = _dev(a["X"]), _dev(a["bias"])
    _repeat_equal(lambda: qp.qgemm_a8w4_blockwise_f32(X, blob, info, b, -6.0, 6.0))
    _repeat_equal(lambda: qp.qgemm_a8w4_blockq_f32(X, blob, info, b, -6.0, 6.0))


def test_a8w4_rows_agree_across_configurations(qp):
    """Rows 0..15 of an M = 128 call (32-row x 64-channel workgroups) and the same rows as
    an M = 16 call (K split over the waves) agree to the f32 tolerance."""
    print("geometry: A8W4 M=128 vs M=16", flush=True)
    a = synth.a8w4(synth.BASE_SEED + 52, 128, 1024, 4096)
    blob, info = qp.pack_s4(_dev(a["W"]), _dev(a["sw"]))
    X, b = _dev(a["X"]), _dev(a["bias"])
    big = qp.qgemm_a8w4_blockwise_f32(X, blob, info, b, -6.0, 6.0).cpu().numpy()
    small = qp.qgemm_a8w4_blockwise_f32(X[:16].contiguous(), blob, info, b, -6.0,
                                        6.0).cpu().numpy()
    err = np.abs(small.astype(np.float64) - big[:16]) / np.maximum(1.0, np.abs(big[:16]))
    assert (err <= 1e-5).all(), err.max()


def test_block_int8_and_channel_blocked_conv_repeat_bitwise(qp):
    print("determinism: block-quantized int8 GEMM and conv", flush=True)
    rng = np.random.default_rng(62)
    N, K = 4096, 4096
    W = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (N, K // 128)).astype(np.float32)
    blob, info = qp.pack_s8_blockwise(_dev(W), _dev(sw), block=128)
    for M in (1, 16, 64):
        X = _dev(rng.standard_normal((M, K)).astype(np.float32))
        _repeat_equal(lambda: qp.qgemm_a8w8_blockwise_f32(X, blob, info, None, -6.0, 6.0))
    Wc = rng.integers(-127, 128, (64, 64, 3, 3)).astype(np.int8)
    swc = rng.uniform(1e-4, 1e-3, (64, 1)).astype(np.float32)
    bc, ic = qp.pack_s8_blockwise(_dev(Wc), _dev(swc), block=64)
    Xc = _dev(rng.integers(-128, 128, (1, 56, 56, 64)).astype(np.int8))   # the K-split tiles
    _repeat_equal(lambda: qp.qconv2d_s8_blockwise_f32(Xc, 0.05, 7, bc, ic, 3, 3, (1, 1),
                                                      (1, 1, 1, 1), (1, 1), None, 0.0, 6.0))
