"""GPU parity of the INT8 GEMM (+ zero-point correction and requantizing or raw
INT32 epilogue) and of the im2col convolution against the oracle: bit-exact
for every int8 and int32 output."""
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


def _run_gemm_case(qp, orc, A, zA, sA, B_kn, zB, sB, bias, s_out, zp_out, relu, per_channel):
    """GPU int8 and int32 outputs vs oracle O1 + O3 for B given as [K, N]."""
    N = B_kn.shape[1]
    zBv = np.broadcast_to(np.asarray(zB, np.int32), (N,)).copy()
    sBv = np.broadcast_to(np.asarray(sB, np.float32), (N,)).copy()
    if per_channel:
        blob, info = qp.pack_s8(_dev(B_kn), scales=_dev(sBv), zero_points=_dev(zBv), k_axis=0, n_axis=1)
    else:
        blob, info = qp.pack_s8(_dev(B_kn), scale=float(sBv[0]), zero_point=int(zBv[0]), k_axis=0,
                                n_axis=1)
    mab = int(np.abs(bias).max()) if bias is not None else 0
    dA = _dev(A)
    dbias = None if bias is None else _dev(bias)
    c32 = qp.qgemm_s8s8_requant(dA, sA, zA, blob, info, dbias, mab, out_dtype="s32")
    c8 = qp.qgemm_s8s8_requant(dA, sA, zA, blob, info, dbias, mab, s_out, zp_out, relu, out_dtype="s8")
    acc = orc.gemm_affine(A, zA, B_kn, zBv, bias)
    want8, _ = orc.requant_matrix(acc, sA, sBv, s_out, zp_out, relu)
    _first_diff(_host(c32), acc.astype(np.int32), "int32 accumulator")
    _first_diff(_host(c8), want8, "int8 output", acc)


def test_gemm_affine_per_tensor_worked_shape(qp, orc):
    d = synth.gemm_affine_per_tensor()
    _run_gemm_case(qp, orc, d["A"], d["zA"], d["sA"], d["B"], d["zB"], d["sB"], d["bias"],
                   d["s_out"], d["zp_out"], d["relu"], per_channel=False)


def test_gemm_physical_strides(qp, orc):
    """Logical N=70 inside a 128-byte physical row of B, A with lda=160 and an
    output with ldc=96."""
    import torch
    d = synth.gemm_affine_per_tensor()
    Bbig = np.zeros((129, 128), np.int8)
    Bbig[:, :70] = d["B"]
    blob, info = qp.pack_s8(_dev(Bbig)[:, :70], scale=d["sB"], zero_point=d["zB"], k_axis=0, n_axis=1)
    Abig = np.zeros((130, 160), np.int8)
    Abig[:, :129] = d["A"]
    dA = _dev(Abig)[:, :129]
    out = torch.full((130, 96), 77, dtype=torch.int8, device="cuda")
    qp.qgemm_s8s8_requant(dA, d["sA"], d["zA"], blob, info, _dev(d["bias"]), 1000, d["s_out"],
                          d["zp_out"], False, out=out[:, :70])
    acc = orc.gemm_affine(d["A"], d["zA"], d["B"], d["zB"], d["bias"])
    want, _ = orc.requant_matrix(acc, d["sA"], d["sB"], d["s_out"], d["zp_out"], False)
    got = _host(out)
    _first_diff(got[:, :70], want, "strided int8 output", acc)
    assert (got[:, 70:] == 77).all(), "wrote outside the logical output"


@pytest.mark.parametrize("seed", range(12))
def test_gemm_random_small_shapes(qp, orc, seed):
    rng = np.random.default_rng(100 + seed)
    M, N, K = (int(x) for x in rng.integers(1, 71, 3))
    if seed % 3 == 0:
        K = int(rng.integers(64, 400))
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-128, 128, (K, N)).astype(np.int8)
    per_channel = bool(seed % 2)
    zA = int(rng.integers(-128, 128))
    zB = rng.integers(-20, 20, N).astype(np.int32) if per_channel else int(rng.integers(-20, 20))
    sB = rng.uniform(0.001, 0.02, N).astype(np.float32) if per_channel else 0.01
    bias = rng.integers(-5000, 5001, N).astype(np.int32) if seed % 4 != 1 else None
    _run_gemm_case(qp, orc, A, zA, 0.02, B, zB, sB, bias, float(rng.uniform(0.05, 2.0)),
                   int(rng.integers(-128, 128)), bool(seed % 3 == 1), per_channel)


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (513, 129, 384), (256, 256, 640), (1, 300, 512)])
def test_gemm_multi_tile_shapes(qp, orc, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (K, N)).astype(np.int8)
    sB = rng.uniform(0.001, 0.01, N).astype(np.float32)
    bias = rng.integers(-1000, 1001, N).astype(np.int32)
    _run_gemm_case(qp, orc, A, 0, 0.01, B, 0, sB, bias, 1.0, 0, False, True)


def test_gemm_int32_bound_is_reached_exactly(qp, orc):
    K = 129
    A = np.full((3, K), -128, np.int8)
    B = np.full((K, 5), 127, np.int8)
    _run_gemm_case(qp, orc, A, 127, 1.0, B, -128, 1e-6, None, 1.0, 0, False, False)


def test_gemm_large_full_size(qp, orc, large_gemm):
    """The 8192^3 per-channel GEMM, in the launch configuration the benchmark
    times: every int32 accumulator against the fp64-matmul formulation of the
    oracle (O1), every int8 output against O3 applied to those accumulators,
    and the fp64 formulation itself against the scalar O1 loops at sampled
    points."""
    d, acc = large_gemm
    print("8192^3 GEMM, int32 and int8 outputs", flush=True)
    blob, info = qp.pack_s8(_dev(d["W"]), scales=_dev(d["s_w"]))
    dA = _dev(d["A"])
    c32 = _host(qp.qgemm_s8s8_requant(dA, d["sA"], d["zA"], blob, info, out_dtype="s32"))
    _first_diff(c32, acc.astype(np.int32), "int32 accumulators")
    del c32
    c8 = _host(qp.qgemm_s8s8_requant(dA, d["sA"], d["zA"], blob, info, None, 0, d["s_out"],
                                     d["zp_out"], False, out_dtype="s8"))
    want8, _ = orc.requant_matrix(acc, d["sA"], d["s_w"], d["s_out"], d["zp_out"], False)
    _first_diff(c8, want8, "int8 outputs", acc)
    rng = np.random.default_rng(0)
    ms, ns = rng.integers(0, 8192, 2048), rng.integers(0, 8192, 2048)
    pts = orc.gemm_affine_points(ms, ns, d["A"], 0, d["W"], 0, b_is_nk=True)
    assert np.array_equal(acc[ms, ns], pts)


def test_gemm_deterministic_repeats(qp):
    d = synth.gemm_affine_per_tensor(M=700, N=300, K=1000)
    blob, info = qp.pack_s8(_dev(d["B"]), scale=0.01, zero_point=-5, k_axis=0, n_axis=1)
    dA = _dev(d["A"])
    first = _host(qp.qgemm_s8s8_requant(dA, 0.02, 3, blob, info, _dev(d["bias"]), 1000, 0.5, -2))
    for _ in range(10):
        again = _host(qp.qgemm_s8s8_requant(dA, 0.02, 3, blob, info, _dev(d["bias"]), 1000, 0.5, -2))
        assert np.array_equal(first, again)


# ------------------------------------------------------------------ conv
def test_im2col_matches_oracle(qp, orc):
    c = synth.conv3x3_nhwc()
    col = _host(qp.qim2col_s8(_dev(c["X"]), c["zp_in"], 3, 3, c["stride"], c["pad"]))
    want = orc.im2col(c["X"], c["zp_in"], 3, 3, c["stride"], c["pad"])
    _first_diff(col[:, :want.shape[1]], want, "im2col")
    assert not col[:, want.shape[1]:].any()


@pytest.mark.parametrize("geom", [
    dict(NB=1, H=9, W=7, C=5, OC=6, KH=3, KW=3, stride=(1, 1), pad=(1, 1, 1, 1)),
    dict(NB=2, H=10, W=11, C=16, OC=20, KH=3, KW=2, stride=(2, 1), pad=(0, 1, 2, 0)),
    dict(NB=1, H=6, W=6, C=32, OC=7, KH=1, KW=1, stride=(1, 1), pad=(0, 0, 0, 0)),
])
def test_im2col_general_geometry(qp, orc, geom):
    rng = np.random.default_rng(geom["C"])
    X = rng.integers(-128, 128, (geom["NB"], geom["H"], geom["W"], geom["C"])).astype(np.int8)
    col = _host(qp.qim2col_s8(_dev(X), -3, geom["KH"], geom["KW"], geom["stride"], geom["pad"]))
    want = orc.im2col(X, -3, geom["KH"], geom["KW"], geom["stride"], geom["pad"])
    _first_diff(col[:, :want.shape[1]], want, "im2col general")


def _conv_case(qp, orc, X, zp_in, s_in, Wt, s_w, bias, stride, pad, s_out, zp_out, relu):
    OC = Wt.shape[0]
    KH, KW = Wt.shape[2], Wt.shape[3]
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(s_w))
    mab = int(np.abs(bias).max()) if bias is not None else 0
    dX = _dev(X)
    dbias = None if bias is None else _dev(bias)
    y32 = _host(qp.qconv2d_s8_im2col(dX, s_in, zp_in, blob, info, KH, KW, stride, pad, dbias, mab,
                                     out_dtype="s32"))
    y8 = _host(qp.qconv2d_s8_im2col(dX, s_in, zp_in, blob, info, KH, KW, stride, pad, dbias, mab,
                                    s_out, zp_out, relu))
    acc = orc.conv2d_direct(X, zp_in, Wt, stride, pad, bias)
    want8, _ = orc.requant_matrix(acc.reshape(-1, OC), s_in, s_w, s_out, zp_out, relu)
    _first_diff(y32, acc.astype(np.int32), "conv int32")
    _first_diff(y8.reshape(-1, OC), want8, "conv int8", acc.reshape(-1, OC))


def test_conv3x3_workload(qp, orc):
    c = synth.conv3x3_nhwc()
    _conv_case(qp, orc, c["X"], c["zp_in"], c["s_in"], c["W"], c["s_w"], c["bias"], c["stride"],
               c["pad"], c["s_out"], c["zp_out"], c["relu"])


@pytest.mark.parametrize("seed", range(4))
def test_conv_random_geometry(qp, orc, seed):
    rng = np.random.default_rng(500 + seed)
    NB, H, W = int(rng.integers(1, 3)), int(rng.integers(3, 15)), int(rng.integers(3, 15))
    C, OC = int(rng.choice([3, 8, 16, 24])), int(rng.integers(1, 40))
    KH, KW = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    stride = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    pad = tuple(int(rng.integers(0, k)) for k in (KH, KW, KH, KW))
    X = rng.integers(-128, 128, (NB, H, W, C)).astype(np.int8)
    Wt = rng.integers(-127, 128, (OC, C, KH, KW)).astype(np.int8)
    s_w = rng.uniform(0.001, 0.01, OC).astype(np.float32)
    bias = rng.integers(-1000, 1001, OC).astype(np.int32)
    _conv_case(qp, orc, X, int(rng.integers(-128, 128)), 0.05, Wt, s_w, bias, stride, pad, 0.1,
               int(rng.integers(-10, 10)), bool(seed % 2))
