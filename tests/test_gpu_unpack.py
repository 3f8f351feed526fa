"""GPU checks of qunpack_weights (logical values, scales, zero points and
dequantized weights read back out of a blob) and of saving a blob to bytes
and restoring it: bit-exact against the logical inputs and oracle O9, and
the restored blob gives the same GEMM / A8W4 outputs."""
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


@pytest.mark.parametrize("N,K,per_channel", [(70, 129, True), (1, 64, False), (130, 300, True),
                                             (33, 1, True)])
def test_unpack_int8_roundtrip(qp, orc, N, K, per_channel):
    rng = np.random.default_rng(N * 1000 + K)
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    z = rng.integers(-30, 31, N).astype(np.int32)
    if per_channel:
        blob, info = qp.pack_s8(_dev(W), scales=_dev(s), zero_points=_dev(z))
    else:
        s[:] = s[0]
        z[:] = z[0]
        blob, info = qp.pack_s8(_dev(W), scale=float(s[0]), zero_point=int(z[0]))
    w, sc, zp, dq = qp.qunpack_weights(blob, info, dequant=True)
    assert np.array_equal(_host(w), W)
    assert np.array_equal(_host(sc), s) and np.array_equal(_host(zp), z)
    assert np.array_equal(_host(dq), orc.dequant_weights_s8(W, s, z))
    # a channel range
    n0, cnt = N // 3, max(1, N // 2)
    w2, sc2, zp2, dq2 = qp.qunpack_weights(blob, info, n0, cnt, dequant=True)
    assert np.array_equal(_host(w2), W[n0:n0 + cnt]) and np.array_equal(_host(sc2), s[n0:n0 + cnt])


def test_unpack_int8_conv_weights_in_k_order(qp):
    """OIHW weights come back as [OC, K] in the packed K order (ky, kx, ic)."""
    rng = np.random.default_rng(3)
    Wt = rng.integers(-127, 128, (20, 16, 3, 2)).astype(np.int8)
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(np.full(20, 0.01, np.float32)))
    w, _, _, _ = qp.qunpack_weights(blob, info)
    assert np.array_equal(_host(w), Wt.transpose(0, 2, 3, 1).reshape(20, -1))


@pytest.mark.parametrize("N,K", [(48, 4096), (17, 160), (4096, 4096)])
def test_unpack_int4_roundtrip(qp, orc, N, K):
    rng = np.random.default_rng(N + K)
    W = rng.integers(-8, 8, (N, K)).astype(np.int8)
    G = (K + 31) // 32
    sw = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    blob, info = qp.pack_s4(_dev(W), _dev(sw))
    w, sc, zp, dq = qp.qunpack_weights(blob, info, dequant=True)
    assert zp is None
    assert np.array_equal(_host(w), W) and np.array_equal(_host(sc), sw)
    assert np.array_equal(_host(dq), orc.dequant_weights_s4(W, sw, 32))


def test_unpack_rejects_bad_requests(qp):
    import torch
    rng = np.random.default_rng(5)
    W4 = rng.integers(-8, 8, (16, 64)).astype(np.int8)
    blob, info = qp.pack_s4(_dev(W4), _dev(np.full((16, 2), 0.01, np.float32)))
    zp = torch.empty(16, dtype=torch.int32, device="cuda")
    import ctypes as C
    st = qp._lib.qunpack_weights(C.byref(info), qp._ptr(blob), 0, 16, None, 64, None, 2,
                                 qp._ptr(zp), None, 64, qp._stream())
    assert st == qp.QP_EINVAL
    with pytest.raises(qp.QPackError):
        qp.qunpack_weights(blob, info, 10, 7)


def test_blob_save_restore_int8(qp, orc, tmp_path):
    d = synth.gemm_affine_per_tensor()
    blob, info = qp.pack_s8(_dev(d["B"]), scale=d["sB"], zero_point=d["zB"], k_axis=0, n_axis=1)
    path = tmp_path / "w.qpk"
    path.write_bytes(qp.blob_to_bytes(blob))
    blob2, info2 = qp.blob_from_bytes(path.read_bytes())
    assert np.array_equal(_host(blob2), _host(blob))
    for f in ("format", "N", "K", "Npad", "Kpad", "total_bytes", "has_zero_points"):
        assert getattr(info2, f) == getattr(info, f), f
    dA, db = _dev(d["A"]), _dev(d["bias"])
    c1 = _host(qp.qgemm_s8s8_requant(dA, d["sA"], d["zA"], blob, info, db, 1000, d["s_out"],
                                     d["zp_out"]))
    c2 = _host(qp.qgemm_s8s8_requant(dA, d["sA"], d["zA"], blob2, info2, db, 1000, d["s_out"],
                                     d["zp_out"]))
    assert np.array_equal(c1, c2)
    acc = orc.gemm_affine(d["A"], d["zA"], d["B"], d["zB"], d["bias"])
    want, _ = orc.requant_matrix(acc, d["sA"], d["sB"], d["s_out"], d["zp_out"], False)
    assert np.array_equal(c2, want)


def test_blob_save_restore_int4_and_corruption(qp, orc):
    g = synth.a8w4(0x51A7E0 + 9, 3, 96, 256)
    blob, info = qp.pack_s4(_dev(g["W"]), _dev(g["sw"]))
    data = qp.blob_to_bytes(blob)
    blob2, info2 = qp.blob_from_bytes(data)
    X, b = _dev(g["X"]), _dev(g["bias"])
    y1 = _host(qp.qgemm_a8w4_blockwise_f32(X, blob, info, b, -6.0, 6.0))
    y2 = _host(qp.qgemm_a8w4_blockwise_f32(X, blob2, info2, b, -6.0, 6.0))
    assert np.array_equal(y1, y2)
    bad = bytearray(data)
    bad[0] ^= 0xFF                     # magic
    with pytest.raises(qp.QPackError):
        qp.blob_from_bytes(bytes(bad))
    bad = bytearray(data)
    bad[40] ^= 0x01                    # Kpad: geometry no longer consistent
    with pytest.raises(qp.QPackError):
        qp.blob_from_bytes(bytes(bad))
    with pytest.raises(qp.QPackError):
        qp.blob_from_bytes(data[:info.total_bytes - 1])
