"""Reusing packed buffers (tract's new_packed_buffer / repack_tensor_view):
qrepack_weights refills an existing blob in place -- byte-identical to a
fresh pack of the new weights, the GEMM then follows the new weights
(bit-exact against the oracle) -- and refuses weights of another shape or
format, leaving the blob as it was.  The dynamic-quantization buffers of
the activations are refilled per call the same way."""
import numpy as np
import pytest

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


def _bytes(blob):
    import torch
    torch.cuda.synchronize()
    return blob.cpu().numpy().copy()


def test_repack_int8_in_place_then_gemm(qp, orc):
    print("repack int8 70x129", flush=True)
    rng = np.random.default_rng(11)
    N, K, M = 70, 129, 33
    W1 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    W2 = rng.integers(-128, 128, (N, K)).astype(np.int8)
    s1 = rng.uniform(0.001, 0.01, N).astype(np.float32)
    s2 = rng.uniform(0.001, 0.01, N).astype(np.float32)
    z2 = rng.integers(-5, 6, N).astype(np.int32)
    blob, info = qp.pack_s8(_dev(W1), scales=_dev(s1))
    ptr = blob.data_ptr()
    assert info.has_zero_points == 0
    b2, i2 = qp.pack_s8(_dev(W2), scales=_dev(s2), zero_points=_dev(z2), into=(blob, info))
    assert b2 is blob and i2 is info and blob.data_ptr() == ptr
    assert info.has_zero_points == 1
    fresh, finfo = qp.pack_s8(_dev(W2), scales=_dev(s2), zero_points=_dev(z2))
    assert np.array_equal(_bytes(blob)[:info.total_bytes], _bytes(fresh)[:finfo.total_bytes])
    assert info.as_dict() == finfo.as_dict()
    # the GEMM reads the refilled blob
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    bias = rng.integers(-1000, 1001, N).astype(np.int32)
    y = qp.qgemm_s8s8_requant(_dev(A), 0.02, 3, blob, info, _dev(bias), 1000, 0.5, -2,
                              False).cpu().numpy()
    acc = orc.gemm_affine(A, 3, W2, z2, bias, b_is_nk=True)
    want, _ = orc.requant_matrix(acc, 0.02, s2, 0.5, -2, False)
    assert np.array_equal(y, want)


def test_repack_int4_and_block_int8(qp, orc):
    print("repack int4 / block-quantized int8", flush=True)
    rng = np.random.default_rng(12)
    N, K = 96, 300
    W1 = rng.integers(-8, 8, (N, K)).astype(np.int8)
    W2 = rng.integers(-8, 8, (N, K)).astype(np.int8)
    G = (K + 31) // 32
    sw1 = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    sw2 = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    for kw in ({}, {"scale_dtype": "bf16"}):
        blob, info = qp.pack_s4(_dev(W1), _dev(sw1), **kw)
        qp.pack_s4(_dev(W2), _dev(sw2), into=(blob, info), **kw)
        fresh, _ = qp.pack_s4(_dev(W2), _dev(sw2), **kw)
        assert np.array_equal(_bytes(blob), _bytes(fresh))
    off = rng.uniform(-0.01, 0.01, (N, G)).astype(np.float32)
    blob, info = qp.pack_s4(_dev(W1), _dev(sw1), offsets=_dev(off))
    qp.pack_s4(_dev(W2), _dev(sw2), offsets=_dev(off), into=(blob, info))
    fresh, _ = qp.pack_s4(_dev(W2), _dev(sw2), offsets=_dev(off))
    assert np.array_equal(_bytes(blob), _bytes(fresh))
    V1 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    V2 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sb = rng.uniform(1e-4, 1e-3, (N, (K + 63) // 64)).astype(np.float32)
    blob, info = qp.pack_s8_blockwise(_dev(V1), _dev(sb), block=64)
    qp.pack_s8_blockwise(_dev(V2), _dev(sb), block=64, into=(blob, info))
    fresh, _ = qp.pack_s8_blockwise(_dev(V2), _dev(sb), block=64)
    assert np.array_equal(_bytes(blob), _bytes(fresh))


def test_repack_refuses_another_shape_or_format(qp):
    print("repack mismatches", flush=True)
    rng = np.random.default_rng(13)
    W = rng.integers(-127, 128, (70, 129)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, 70).astype(np.float32)
    blob, info = qp.pack_s8(_dev(W), scales=_dev(s))
    before, dict_before = _bytes(blob), info.as_dict()
    bad = [lambda: qp.pack_s8(_dev(W[:, :128]), scales=_dev(s), into=(blob, info)),   # K
           lambda: qp.pack_s8(_dev(W[:69]), scales=_dev(s[:69]), into=(blob, info)),  # N
           lambda: qp.pack_s4(_dev(np.zeros((70, 129), np.int8)),                     # format
                              _dev(np.ones((70, 5), np.float32)), into=(blob, info)),
           lambda: qp.pack_s8(_dev(W), scale=0.01, into=(blob, info))]               # scheme
    for f in bad:
        with pytest.raises(qp.QPackError, match="qrepack_weights: the buffer holds"):
            f()
    assert np.array_equal(_bytes(blob), before) and info.as_dict() == dict_before


def test_activation_buffers_refilled_per_call(qp, orc):
    """One set of quantized-activation buffers, refilled for each new input
    (the A8W4 prequant path): every call matches a fresh quantization and
    the product follows the newest input."""
    import torch
    import synth
    print("activation buffer reuse", flush=True)
    a = synth.a8w4(synth.BASE_SEED + 21, 8, 256, 512)
    blob4, info4 = qp.pack_s4(_dev(a["W"]), _dev(a["sw"]))
    q = torch.empty((8, info4.Kpad), dtype=torch.int8, device="cuda")
    sa = torch.empty(8, dtype=torch.float32, device="cuda")
    za = torch.empty(8, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(14)
    for step in range(3):
        X = rng.standard_normal((8, 512)).astype(np.float32)
        qp.qquantize_rows_s8(_dev(X), q=q, row_scale=sa, row_zp=za)
        qf, sf, zf = qp.qquantize_rows_s8(_dev(X))
        assert np.array_equal(q[:, :512].cpu().numpy(), qf.cpu().numpy())
        assert np.array_equal(sa.cpu().numpy(), sf.cpu().numpy())
        assert np.array_equal(za.cpu().numpy(), zf.cpu().numpy())
        y = qp.qgemm_a8w4_prequant_f32(q, sa, za, blob4, info4, _dev(a["bias"]), -6.0,
                                       6.0).cpu().numpy()
        want = orc.a8w4_forward(X, a["W"], a["sw"], a["bias"], -6.0, 6.0)
        err = np.abs(y.astype(np.float64) - want) / np.maximum(1.0, np.abs(want))
        assert (err <= 1e-5).all(), (step, err.max())
