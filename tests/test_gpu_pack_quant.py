"""GPU parity of the weight packer and the dynamic row quantizer against the
oracle: bit-exact.  Calls go through the C ABI (the ctypes binding)."""
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


def _first_diff(got, want, what):
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s: gpu=%s oracle=%s"
                             % (what, len(bad), i, got[i], want[i]))


# ------------------------------------------------------------------ S8 pack
@pytest.mark.parametrize("N,K,src", [(70, 129, "kn"), (64, 576, "nk"), (8, 8, "nk"), (1, 1, "kn"),
                                     (130, 64, "kn"), (257, 200, "nk"), (65, 1000, "nk")])
def test_pack_s8_matches_reference_blob(qp, orc, N, K, src):
    rng = np.random.default_rng(N * 1000 + K)
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    sc = rng.uniform(0.001, 0.01, N).astype(np.float32)
    zp = rng.integers(-5, 5, N).astype(np.int32)
    want = orc.pack_s8_ref(W, sc, zp, per_channel=True)
    if src == "kn":
        blob, info = qp.pack_s8(_dev(W.T), scales=_dev(sc), zero_points=_dev(zp), k_axis=0, n_axis=1)
    else:
        blob, info = qp.pack_s8(_dev(W), scales=_dev(sc), zero_points=_dev(zp))
    got = _host(blob)[: want.size]
    _first_diff(got, want, "int8 blob")
    assert info.total_bytes == want.size and info.has_zero_points == int(zp.any())


def test_pack_s8_per_tensor_and_strided_view(qp, orc):
    rng = np.random.default_rng(3)
    big = rng.integers(-128, 128, (129, 128)).astype(np.int8)   # physical row of 128 bytes
    B = big[:, :70]                                              # logical [K=129, N=70]
    want = orc.pack_s8_ref(B.T, np.array([0.01], np.float32), np.array([-5], np.int32),
                           per_channel=False)
    t = _dev(big)[:, :70]
    blob, info = qp.pack_s8(t, scale=0.01, zero_point=-5, k_axis=0, n_axis=1)
    _first_diff(_host(blob)[: want.size], want, "per-tensor strided blob")
    assert info.has_zero_points == 1


def test_pack_s8_conv_oihw(qp, orc):
    c = synth.conv3x3_nhwc()
    Bnk = c["W"].transpose(0, 2, 3, 1).reshape(64, -1)   # K order (kh, kw, ic)
    want = orc.pack_s8_ref(Bnk, c["s_w"])
    blob, info = qp.pack_s8(_dev(c["W"]), scales=_dev(c["s_w"]))
    _first_diff(_host(blob)[: want.size], want, "OIHW blob")
    assert (info.N, info.K, info.Kpad) == (64, 576, 576)


# ------------------------------------------------------------------ S4 pack
@pytest.mark.parametrize("N,K", [(4096, 4096), (5, 100), (64, 32), (130, 4000), (1, 33)])
def test_pack_s4_matches_reference_blob(qp, orc, N, K):
    rng = np.random.default_rng(N + K)
    W = rng.integers(-8, 8, (N, K)).astype(np.int8)
    G = (K + 31) // 32
    sw = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    want = orc.pack_s4_ref(W, sw, 32)
    blob, info = qp.pack_s4(_dev(W), _dev(sw))
    got = _host(blob)[: want.size]
    _first_diff(got, want, "int4 blob")
    assert info.total_bytes == want.size


def test_pack_s4_flags_out_of_range_values(qp):
    W = np.zeros((3, 32), np.int8)
    W[1, 7] = 9
    blob, info = qp.pack_s4(_dev(W), _dev(np.ones((3, 1), np.float32)))
    hdr = _host(blob)[:256]
    assert hdr[108:112].view(np.int32)[0] != 0
    import conv_qpack_weights_amd as qpk
    with pytest.raises(qpk.QPackError):
        qpk.qp_packed_info_from_header(hdr.tobytes())


def test_blob_header_round_trip(qp):
    rng = np.random.default_rng(5)
    W = rng.integers(-128, 128, (70, 129)).astype(np.int8)
    blob, info = qp.pack_s8(_dev(W), scales=_dev(np.full(70, 0.01, np.float32)))
    back = qp.qp_packed_info_from_header(_host(blob)[:256].tobytes())
    for f in ["format", "N", "K", "Npad", "Kpad", "data_off", "scale_off", "sum_off", "zp_off",
              "total_bytes", "has_zero_points", "scale_min", "scale_max"]:
        assert getattr(back, f) == getattr(info, f), f


# ------------------------------------------------------------------ S3 quantizer
def _quant_rows_cases():
    rng = np.random.default_rng(9)
    d3 = synth.a8w4_gemv()
    d4 = synth.a8w4_gemm(16)
    d5 = synth.a8w4_gemm(128)
    rows = [d3["X"], d4["X"], d5["X"],
            rng.standard_normal((3, 777)).astype(np.float32),
            np.zeros((2, 64), np.float32),
            np.abs(rng.standard_normal((2, 100))).astype(np.float32),
            -np.abs(rng.standard_normal((2, 100))).astype(np.float32),
            np.array([[0.0, 255.0] + [j + 0.5 for j in range(0, 254)]], np.float32),
            (rng.standard_normal((1, 1)) * 3).astype(np.float32)]
    return rows


@pytest.mark.parametrize("case", range(9))
def test_quantize_rows_bit_exact(qp, orc, case):
    X = _quant_rows_cases()[case]
    q, s, z = qp.qquantize_rows_s8(_dev(X))
    wq, ws, wz = orc.quantize_rows_s8(X)
    _first_diff(_host(s), ws, "row scale")
    _first_diff(_host(z), wz, "row zero point")
    _first_diff(_host(q), wq, "row codes")


def _sym_rows_cases():
    rng = np.random.default_rng(19)
    return [synth.a8w4_gemm(16)["X"],
            rng.standard_normal((3, 4099)).astype(np.float32) * 7,
            np.zeros((2, 64), np.float32),
            np.array([[127.0 / 128.0] + [(j + 0.5) / 128.0 for j in range(-127, 127)]],
                     np.float32),
            (rng.standard_normal((1, 1)) * 3).astype(np.float32)]


@pytest.mark.parametrize("case", range(5))
def test_quantize_rows_sym_bit_exact(qp, orc, case):
    X = _sym_rows_cases()[case]
    q, s = qp.qquantize_rows_s8_sym(_dev(X))
    wq, ws = orc.quantize_rows_s8_sym(X)
    _first_diff(_host(s), ws, "sym row scale")
    _first_diff(_host(q), wq, "sym row codes")


def test_quantize_rows_strided_input(qp, orc):
    import torch
    rng = np.random.default_rng(10)
    big = rng.standard_normal((5, 300)).astype(np.float32)
    X = _dev(big)[:, :257]
    q = torch.empty((5, 272), dtype=torch.int8, device="cuda")
    q, s, z = qp.qquantize_rows_s8(X, q=q)
    wq, ws, wz = orc.quantize_rows_s8(big[:, :257])
    _first_diff(_host(q)[:, :257], wq, "strided codes")
    _first_diff(_host(s), ws, "strided scales")
