"""GPU parity of the INT8 GEMM with f32 output (dequantize, f32 bias, clamp)
against the oracle's exact accumulator followed by O8.

Tolerance: |gpu - oracle| <= 1e-5 * max(1, |oracle|), and the bound the
arithmetic gives: the kernel rounds sA*sB[n] and the int32 accumulator to
f32 and then does one fused multiply-add, so its error is at most
3 * 2^-24 * (|sA*sB*acc| + |bias|) away from the fp64 value (which the oracle
rounds once more, half an ulp of the result)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


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


def _check_f32(got, want, acc, sA, sB, bias, what):
    N = want.shape[1]
    sBv = np.broadcast_to(np.asarray(sB, np.float64), (N,))
    bv = np.zeros(N) if bias is None else np.asarray(bias, np.float64)
    mag = np.abs(float(sA) * sBv[None, :] * acc.astype(np.float64)) + np.abs(bv)[None, :]
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bar = 1e-5 * np.maximum(1.0, np.abs(want.astype(np.float64)))
    derived = 3 * U * mag + U * np.abs(want.astype(np.float64))
    bad = np.argwhere((err > bar) | (err > derived))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d outside tolerance, first at %s: gpu=%r oracle=%r acc=%d"
                             % (what, len(bad), i, got[i], want[i], acc[i]))


def _case(qp, orc, A, zA, sA, B_kn, zB, sB, bias, lo, hi, per_channel):
    N = B_kn.shape[1]
    zBv = np.broadcast_to(np.asarray(zB, np.int32), (N,)).copy()
    sBv = np.broadcast_to(np.asarray(sB, np.float32), (N,)).copy()
    if per_channel:
        blob, info = qp.pack_s8(_dev(B_kn), scales=_dev(sBv), zero_points=_dev(zBv), k_axis=0,
                                n_axis=1)
    else:
        blob, info = qp.pack_s8(_dev(B_kn), scale=float(sBv[0]), zero_point=int(zBv[0]),
                                k_axis=0, n_axis=1)
    y = _host(qp.qgemm_s8s8_dequant_f32(_dev(A), sA, zA, blob, info,
                                         None if bias is None else _dev(bias), lo, hi))
    acc = orc.gemm_affine(A, zA, B_kn, zBv, None)
    want = orc.dequant_matrix_f32(acc, sA, sBv, bias, lo, hi)
    _check_f32(y, want, acc, sA, sBv, bias, "f32 output")
    return y, want


def test_f32_worked_shape_per_tensor(qp, orc):
    d = synth.gemm_affine_per_tensor()
    rng = np.random.default_rng(5)
    bias = rng.uniform(-3, 3, d["B"].shape[1]).astype(np.float32)
    _case(qp, orc, d["A"], d["zA"], d["sA"], d["B"], d["zB"], d["sB"], bias, -np.inf, np.inf,
          False)


@pytest.mark.parametrize("seed", range(10))
def test_f32_random_small_shapes(qp, orc, seed):
    rng = np.random.default_rng(300 + seed)
    M, N, K = (int(x) for x in rng.integers(1, 71, 3))
    if seed % 3 == 0:
        K = int(rng.integers(64, 400))
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-128, 128, (K, N)).astype(np.int8)
    per_channel = bool(seed % 2)
    zA = int(rng.integers(-128, 128))
    zB = rng.integers(-20, 20, N).astype(np.int32) if per_channel else int(rng.integers(-20, 20))
    sB = rng.uniform(1e-4, 2e-3, N).astype(np.float32) if per_channel else 1e-3
    bias = rng.uniform(-5, 5, N).astype(np.float32) if seed % 4 != 1 else None
    lo, hi = [(-np.inf, np.inf), (0.0, 6.0), (0.0, np.inf), (-1.0, 1.0)][seed % 4]
    _case(qp, orc, A, zA, 0.02, B, zB, sB, bias, lo, hi, per_channel)


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (513, 129, 384), (256, 256, 640),
                                   (1, 300, 512)])
def test_f32_multi_tile_shapes(qp, orc, M, N, K):
    rng = np.random.default_rng(7 * M + N + K)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (K, N)).astype(np.int8)
    sB = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    zB = rng.integers(-8, 8, N).astype(np.int32)
    bias = rng.uniform(-3, 7, N).astype(np.float32)
    y, want = _case(qp, orc, A, 5, 0.01, B, zB, sB, bias, 0.0, 6.0, True)
    # relu6 really clamps on both sides in these cases
    assert (want == 0).any() and (want == 6).any()


def test_f32_clamp_to_single_value(qp, orc):
    rng = np.random.default_rng(11)
    A = rng.integers(-128, 128, (40, 96)).astype(np.int8)
    B = rng.integers(-128, 128, (96, 33)).astype(np.int8)
    y, _ = _case(qp, orc, A, 0, 0.02, B, 0, 0.001, None, 0.75, 0.75, False)
    assert (y == np.float32(0.75)).all()


def test_f32_physical_strides(qp, orc):
    """N=70 inside a 96-float output row; everything past column 70 untouched."""
    import torch
    d = synth.gemm_affine_per_tensor()
    blob, info = qp.pack_s8(_dev(d["B"]), scale=d["sB"], zero_point=d["zB"], k_axis=0, n_axis=1)
    Abig = np.zeros((130, 160), np.int8)
    Abig[:, :129] = d["A"]
    out = torch.full((130, 96), -7.5, dtype=torch.float32, device="cuda")
    bias = np.linspace(-1, 1, 70).astype(np.float32)
    qp.qgemm_s8s8_dequant_f32(_dev(Abig)[:, :129], d["sA"], d["zA"], blob, info, _dev(bias),
                              out=out[:, :70])
    acc = orc.gemm_affine(d["A"], d["zA"], d["B"], d["zB"], None)
    want = orc.dequant_matrix_f32(acc, d["sA"], d["sB"], bias, -np.inf, np.inf)
    got = _host(out)
    _check_f32(got[:, :70], want, acc, d["sA"], d["sB"], bias, "strided f32 output")
    assert (got[:, 70:] == -7.5).all(), "wrote outside the logical output"


def test_f32_large_full_size(qp, orc, large_gemm):
    """The 8192^3 per-channel GEMM with f32 output, in the launch
    configuration the benchmark times: every output against the fp64-matmul
    accumulator followed by O8."""
    d, acc = large_gemm
    print("8192^3 GEMM, f32 output", flush=True)
    rng = np.random.default_rng(12)
    bias = rng.uniform(-1, 1, 8192).astype(np.float32)
    blob, info = qp.pack_s8(_dev(d["W"]), scales=_dev(d["s_w"]))
    y = _host(qp.qgemm_s8s8_dequant_f32(_dev(d["A"]), d["sA"], d["zA"], blob, info, _dev(bias)))
    want = orc.dequant_matrix_f32(acc, d["sA"], d["s_w"], bias, -np.inf, np.inf)
    _check_f32(y, want, acc, d["sA"], d["s_w"], bias, "f32 outputs")


def test_f32_rejects_bad_bounds(qp):
    import torch
    rng = np.random.default_rng(2)
    B = rng.integers(-128, 128, (64, 16)).astype(np.int8)
    blob, info = qp.pack_s8(_dev(B), scale=0.01, zero_point=0, k_axis=0, n_axis=1)
    A = torch.zeros((4, 64), dtype=torch.int8, device="cuda")
    for lo, hi in [(1.0, 0.0), (float("nan"), 1.0), (0.0, float("nan"))]:
        with pytest.raises(Exception):
            qp.qgemm_s8s8_dequant_f32(A, 0.1, 0, blob, info, None, lo, hi)
