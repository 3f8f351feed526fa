"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host -- with a status code
and a message, before any launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def qp():
    import conv_qpack_weights_amd as qp
    return qp


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qpack.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(q\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["qpack_weights", "qpack_weights_size", "qquantize_rows_s8", "qgemm_s8s8_requant",
              "qgemm_a8w4_blockwise_f32", "qconv2d_s8_im2col", "qim2col_s8", "qp_last_error",
              "qp_version", "qp_packed_info_from_header", "qgemm_a8w4_prequant_f32"]:
        assert n in names


def test_library_exports_every_declared_symbol(qp):
    raw = C.CDLL(qp.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(raw, n), "missing export " + n
        assert n in qp.SIGNATURES, "binding lacks " + n
    assert b"gfx950" in qp.lib().qp_version()


def _expect(qp, status, code, needle=None):
    assert status == code, (status, qp.last_error())
    msg = qp.last_error()
    assert msg
    if needle:
        assert needle in msg, msg


def _w8_desc(qp, N=70, K=129, **kw):
    return qp.qtensor(qp.QP_S8, [N, K], [K, 1], **kw)


def test_pack_size_matches_the_reference_geometry(qp, orc):
    for N, K in [(1, 1), (70, 129), (64, 576), (8192, 8192), (65, 63)]:
        nb, al = qp.qpack_weights_size(_w8_desc(qp, N, K), 1, 0)
        assert nb == orc.lib().orc_packed_s8_bytes(N, K) and al == 256
        d4 = qp.qtensor(qp.QP_S4, [N, K], [K, 1], scheme=qp.QP_BLOCKWISE, group_size=32)
        assert qp.qpack_weights_size(d4, 1, 0)[0] == orc.lib().orc_packed_s4_bytes(N, K, 32)


def test_header_parser_reads_the_reference_blob(qp, orc):
    rng = np.random.default_rng(1)
    W = rng.integers(-128, 128, (70, 129)).astype(np.int8)
    blob = orc.pack_s8_ref(W, np.full(70, 0.01, np.float32), np.full(70, -5, np.int32))
    info = qp.qp_packed_info_from_header(blob[:256].tobytes())
    assert (info.format, info.N, info.K, info.Npad, info.Kpad) == (1, 70, 129, 128, 192)
    assert info.total_bytes == blob.size and info.has_zero_points == 1
    # the weight-scale range travels in the header, so a restored blob
    # validates requantization multipliers like a freshly packed one
    assert (info.scale_min, info.scale_max) == (np.float32(0.01), np.float32(0.01))
    norange = bytearray(blob[:256].tobytes())
    norange[112:120] = bytes(8)
    with pytest.raises(qp.QPackError):
        qp.qp_packed_info_from_header(bytes(norange))
    W4 = rng.integers(-8, 8, (5, 100)).astype(np.int8)
    blob4 = orc.pack_s4_ref(W4, np.ones((5, 4), np.float32))
    info4 = qp.qp_packed_info_from_header(blob4[:256].tobytes())
    assert (info4.format, info4.group, info4.Kpad, info4.total_bytes) == (2, 32, 128, blob4.size)
    blob5 = orc.pack_s4_ref(rng.integers(-8, 8, (2, 200)).astype(np.int8), np.ones((2, 7), np.float32))
    info5 = qp.qp_packed_info_from_header(blob5[:256].tobytes())
    assert (info5.Kpad, info5.total_bytes) == (256, blob5.size)
    bad = bytearray(blob[:256].tobytes())
    bad[0] ^= 0xFF
    with pytest.raises(qp.QPackError):
        qp.qp_packed_info_from_header(bytes(bad))
    # an int4 blob deeper than the packer accepts is refused on restore too
    deep = orc.pack_s4_ref(rng.integers(-8, 8, (1, 65537)).astype(np.int8),
                           np.ones((1, 2049), np.float32))
    with pytest.raises(qp.QPackError, match="65536"):
        qp.qp_packed_info_from_header(deep[:256].tobytes())


def test_pack_rejects_bad_descriptors(qp):
    nb, al = C.c_size_t(), C.c_size_t()
    L = qp.lib()
    d = _w8_desc(qp)
    _expect(qp, L.qpack_weights_size(C.byref(d), 0, 0, C.byref(nb), C.byref(al)), qp.QP_EINVAL,
            "permutation")
    d3 = qp.qtensor(qp.QP_S8, [2, 3, 4], None)
    _expect(qp, L.qpack_weights_size(C.byref(d3), 1, 0, C.byref(nb), C.byref(al)), qp.QP_EINVAL)
    d4 = qp.qtensor(qp.QP_S4, [8, 64], [64, 1], scheme=qp.QP_BLOCKWISE, group_size=48)
    _expect(qp, L.qpack_weights_size(C.byref(d4), 1, 0, C.byref(nb), C.byref(al)),
            qp.QP_EUNSUPPORTED, "group size")
    dz = qp.qtensor(qp.QP_S4, [8, 64], [64, 1], scheme=qp.QP_BLOCKWISE, group_size=32,
                    zero_point=3)
    _expect(qp, L.qpack_weights_size(C.byref(dz), 1, 0, C.byref(nb), C.byref(al)),
            qp.QP_EUNSUPPORTED, "zero points")
    dk = qp.qtensor(qp.QP_S4, [8, 65537], [65537, 1], scheme=qp.QP_BLOCKWISE, group_size=32)
    _expect(qp, L.qpack_weights_size(C.byref(dk), 1, 0, C.byref(nb), C.byref(al)),
            qp.QP_EUNSUPPORTED, "65536")
    dr = _w8_desc(qp, rounding=1)
    _expect(qp, L.qpack_weights_size(C.byref(dr), 1, 0, C.byref(nb), C.byref(al)),
            qp.QP_EUNSUPPORTED, "half-to-even")
    info = qp.PackedInfo()
    _expect(qp, L.qpack_weights(C.byref(d), C.c_void_p(FAKE), 1, 0, C.c_void_p(FAKE * 16), 100,
                                C.byref(info), None), qp.QP_ESIZE)
    _expect(qp, L.qpack_weights(C.byref(d), C.c_void_p(FAKE), 1, 0, C.c_void_p(FAKE + 16), 1 << 20,
                                C.byref(info), None), qp.QP_EALIGN)


def _info8(qp, N=70, K=129, has_zp=0, smin=0.001, smax=0.01):
    i = qp.PackedInfo()
    i.format, i.scheme, i.N, i.K = 1, qp.QP_PER_CHANNEL, N, K
    i.Npad, i.Kpad = (N + 63) // 64 * 64, (K + 63) // 64 * 64
    i.has_zero_points, i.scale_min, i.scale_max = has_zp, smin, smax
    i.data_off, i.total_bytes = 256, 1 << 20
    return i


def _gemm(qp, a, info, out, bias=None, mab=0, ws_bytes=1 << 20):
    return qp.lib().qgemm_s8s8_requant(C.byref(a), C.c_void_p(FAKE), C.byref(info),
                                       C.c_void_p(FAKE * 16), bias, mab, C.byref(out), 0,
                                       C.c_void_p(FAKE * 32), C.c_void_p(FAKE * 64), ws_bytes, None)


def test_gemm_rejects_overflow_and_bad_arguments(qp):
    K = 129
    a = qp.qtensor(qp.QP_S8, [130, K], [K, 1], scale=0.02, zero_point=3)
    out = qp.qtensor(qp.QP_S8, [130, 70], [70, 1], scale=0.5, zero_point=-2)
    # [NPU] section 4: K*65025 + |bias| must fit INT32
    limit = 2 ** 31 - 1 - K * 65025
    _expect(qp, _gemm(qp, a, _info8(qp), out, C.c_void_p(FAKE), limit + 1), qp.QP_EOVERFLOW,
            "exceeds INT32")
    big = qp.qtensor(qp.QP_S8, [4, 40000], [40000, 1], scale=0.02)
    _expect(qp, _gemm(qp, big, _info8(qp, K=40000), qp.qtensor(qp.QP_S32, [4, 70], [70, 1])),
            qp.QP_EOVERFLOW)
    _expect(qp, _gemm(qp, a, _info8(qp, K=128), out), qp.QP_EINVAL, "K=")
    f32 = qp.qtensor(qp.QP_F32, [130, 70], [70, 1])
    _expect(qp, _gemm(qp, a, _info8(qp), f32), qp.QP_EUNSUPPORTED)
    sym = qp.qtensor(qp.QP_S8, [130, 70], [70, 1], scale=0.5, qmin=-127)
    _expect(qp, _gemm(qp, a, _info8(qp), sym), qp.QP_EUNSUPPORTED, "[-128,127]")
    _expect(qp, _gemm(qp, a, _info8(qp, smax=1e12), out), qp.QP_EUNSUPPORTED, "multiplier")
    wrong = qp.qtensor(qp.QP_S8, [130, 71], [71, 1], scale=0.5)
    _expect(qp, _gemm(qp, a, _info8(qp), wrong), qp.QP_EINVAL, "output shape")
    kstride = qp.qtensor(qp.QP_S8, [130, K], [1, 130], scale=0.02)
    _expect(qp, _gemm(qp, kstride, _info8(qp), out), qp.QP_EUNSUPPORTED, "K-contiguous")
    # 256x256 tiles with lda = K = 1000 take the padded copy of A: a 0-byte
    # workspace is too small
    wide = qp.qtensor(qp.QP_S8, [4096, 1000], [1000, 1], scale=0.02, zero_point=3)
    wout = qp.qtensor(qp.QP_S8, [4096, 4096], [4096, 1], scale=0.5, zero_point=-2)
    _expect(qp, _gemm(qp, wide, _info8(qp, N=4096, K=1000), wout, ws_bytes=0), qp.QP_ESIZE,
            "workspace")


def test_gemm_workspace_plan(qp):
    """64x64-tile GEMMs up to K = 960 need no workspace (direct loads, or
    activations read byte-exact into LDS with their row sums); deeper or
    larger ones with an odd stride size the padded copy and row sums."""
    L = qp.lib()

    def ws(M, K, N, lda, zp=0):
        n = C.c_size_t()
        a = qp.qtensor(qp.QP_S8, [M, K], [lda, 1])
        assert L.qgemm_s8s8_requant_ws_size(C.byref(a), C.byref(_info8(qp, N=N, K=K, has_zp=zp)),
                                            C.byref(n)) == 0
        return n.value

    assert ws(130, 129, 70, 129) == 0
    assert ws(130, 129, 70, 129, zp=1) == 0
    assert ws(1000, 960, 500, 961, zp=1) == 0
    assert ws(1000, 961, 500, 961) == 1000 * 1024
    assert ws(1000, 961, 500, 961, zp=1) == 1000 * 1024 + 4096
    assert ws(4096, 1000, 4096, 1000) == 4096 * 1024


def test_gemm_overflow_limit_is_inclusive(qp):
    # the largest allowed bound passes validation and fails only at the workspace check
    K = 1000
    a = qp.qtensor(qp.QP_S8, [4096, K], [K, 1], scale=0.02, zero_point=3)
    out = qp.qtensor(qp.QP_S8, [4096, 4096], [4096, 1], scale=0.5, zero_point=-2)
    limit = 2 ** 31 - 1 - K * 65025
    _expect(qp, _gemm(qp, a, _info8(qp, N=4096, K=K), out, C.c_void_p(FAKE), limit, ws_bytes=0),
            qp.QP_ESIZE)


def test_a8w4_quantize_im2col_conv_reject_bad_arguments(qp):
    L = qp.lib()
    i4 = qp.PackedInfo()
    i4.format, i4.N, i4.K, i4.Npad, i4.Kpad, i4.group = 2, 64, 128, 64, 128, 64
    _expect(qp, L.qgemm_a8w4_blockwise_f32(C.c_void_p(FAKE), 1, 128, 128, C.byref(i4),
                                           C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 64,
                                           None, 0, None), qp.QP_EUNSUPPORTED, "group")
    i4.group = 32
    _expect(qp, L.qgemm_a8w4_blockwise_f32(C.c_void_p(FAKE), 1, 100, 128, C.byref(i4),
                                           C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 64,
                                           None, 0, None), qp.QP_EINVAL, "K=")
    _expect(qp, L.qgemm_a8w4_blockwise_f32(C.c_void_p(FAKE), 1, 128, 128, C.byref(i4),
                                           C.c_void_p(FAKE), None, 6.0, -6.0, C.c_void_p(FAKE), 64,
                                           None, 0, None), qp.QP_EINVAL, "clamp")
    _expect(qp, L.qgemm_a8w4_blockwise_f32(C.c_void_p(FAKE), 4, 128, 128, C.byref(i4),
                                           C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 64,
                                           None, 0, None), qp.QP_ESIZE, "workspace")
    i8 = _info8(qp)
    _expect(qp, L.qgemm_a8w4_blockwise_f32(C.c_void_p(FAKE), 1, 129, 129, C.byref(i8),
                                           C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 70,
                                           None, 0, None), qp.QP_EINVAL, "int4")
    _expect(qp, L.qquantize_rows_s8(C.c_void_p(FAKE), 2, 100, 100, C.c_void_p(FAKE), 99,
                                    C.c_void_p(FAKE), C.c_void_p(FAKE), None), qp.QP_EINVAL)
    _expect(qp, L.qim2col_s8(C.c_void_p(FAKE), 1, 8, 8, 4, 0, 3, 3, 1, 1, 1, 1, 1, 1,
                             C.c_void_p(FAKE), 40, None), qp.QP_EINVAL, "multiple of 16")
    _expect(qp, L.qim2col_s8(C.c_void_p(FAKE), 1, 8, 8, 4, 0, 3, 3, 0, 1, 1, 1, 1, 1,
                             C.c_void_p(FAKE), 48, None), qp.QP_EINVAL, "positive")
    x = qp.qtensor(qp.QP_S8, [1, 8, 8, 4], [256, 32, 4, 1], scale=0.05, zero_point=7)
    y = qp.qtensor(qp.QP_S8, [1, 8, 8, 71], None, scale=0.1)
    n = C.c_size_t()
    _expect(qp, L.qconv2d_s8_im2col_ws_size(C.byref(x), C.byref(i8), 3, 3, 1, 1, 1, 1, 1, 1,
                                            C.byref(n)), qp.QP_EINVAL, "KH*KW*C")
    xs = qp.qtensor(qp.QP_S8, [1, 8, 8, 4], [512, 64, 8, 1], scale=0.05)
    i36 = _info8(qp, K=36)
    _expect(qp, L.qconv2d_s8_im2col_ws_size(C.byref(xs), C.byref(i36), 3, 3, 1, 1, 1, 1, 1, 1,
                                            C.byref(n)), qp.QP_EUNSUPPORTED, "contiguous")
    assert L.qconv2d_s8_im2col_ws_size(C.byref(x), C.byref(i36), 3, 3, 1, 1, 1, 1, 1, 1,
                                       C.byref(n)) == qp.QP_OK
    assert n.value >= 64 * 64
    _expect(qp, L.qconv2d_s8_im2col(C.byref(x), C.c_void_p(FAKE), C.byref(i36), C.c_void_p(FAKE),
                                    3, 3, 1, 1, 1, 1, 1, 1, None, 0, C.byref(y), 1,
                                    C.c_void_p(FAKE), C.c_void_p(FAKE * 16), 1 << 20, None),
            qp.QP_EINVAL, "y must be")


def test_blob_geometry_of_the_newer_formats(qp):
    """bf16 scales halve the scale region, asymmetric int4 adds an offset
    region of the scales' size, block-quantized int8 keeps the int8 tiles
    and stores one scale per block."""
    nb, al = C.c_size_t(), C.c_size_t()
    L = qp.lib()
    N, K = 100, 1000

    def size(dtype, scheme, group=32):
        d = qp.qtensor(dtype, [N, K], [K, 1], scheme=scheme, group_size=group)
        assert L.qpack_weights_size(C.byref(d), 1, 0, C.byref(nb), C.byref(al)) == qp.QP_OK, \
            qp.last_error()
        return nb.value

    Npad, Kpad4 = 128, 1024
    def r256(x):
        return (x + 255) // 256 * 256
    data4 = r256(Npad * Kpad4 // 2)
    sc32 = r256(16 * Npad * ((Kpad4 // 32 + 3) // 4))
    assert size(qp.QP_S4, qp.QP_BLOCKWISE) == 256 + data4 + sc32 + r256(4 * Npad)
    assert size(qp.QP_S4, qp.QP_BLOCKWISE_BF16) == 256 + data4 + r256(sc32 // 2) + r256(4 * Npad)
    assert size(qp.QP_S4, qp.QP_BLOCKWISE_ASYM) == 256 + data4 + 2 * sc32 + r256(4 * Npad)
    Kpad8 = 1024
    for g in (64, 128):
        assert size(qp.QP_S8, qp.QP_BLOCKWISE, g) == (256 + r256(Npad * Kpad8) +
                                                      r256(4 * Npad * (Kpad8 // g)) + r256(4 * Npad))
    d = qp.qtensor(qp.QP_S8, [N, K], [K, 1], scheme=qp.QP_BLOCKWISE, group_size=32)
    _expect(qp, L.qpack_weights_size(C.byref(d), 1, 0, C.byref(nb), C.byref(al)),
            qp.QP_EUNSUPPORTED, "64 or 128")


def test_newer_entry_points_reject_bad_arguments(qp):
    L = qp.lib()
    i8 = _info8(qp)
    a = qp.qtensor(qp.QP_S8, [130, 129], [129, 1], scale=0.02, zero_point=3)
    # f32-output GEMM: reversed or NaN clamp bounds, short ldy
    for lo, hi, ldy in [(1.0, 0.0, 70), (float("nan"), 1.0, 70), (0.0, 6.0, 69)]:
        _expect(qp, L.qgemm_s8s8_dequant_f32(C.byref(a), C.c_void_p(FAKE), C.byref(i8),
                                             C.c_void_p(FAKE), None, lo, hi, C.c_void_p(FAKE), ldy,
                                             C.c_void_p(FAKE * 16), 1 << 20, None), qp.QP_EINVAL)
    # per-block quantizer: block 64 unsupported, kpad below K
    _expect(qp, L.qquantize_rows_s8_blocked(C.c_void_p(FAKE), 2, 100, 100, 64, 128,
                                            C.c_void_p(FAKE), 128, C.c_void_p(FAKE),
                                            C.c_void_p(FAKE), 4, None), qp.QP_EUNSUPPORTED)
    _expect(qp, L.qquantize_rows_s8_blocked(C.c_void_p(FAKE), 2, 100, 100, 32, 96,
                                            C.c_void_p(FAKE), 128, C.c_void_p(FAKE),
                                            C.c_void_p(FAKE), 4, None), qp.QP_EINVAL, "kpad")
    # per-block activations refuse asymmetric int4; the int8-blockwise GEMM refuses int4 blobs
    i4 = qp.PackedInfo()
    i4.format, i4.N, i4.K, i4.Npad, i4.Kpad, i4.group = 4, 64, 128, 64, 128, 32
    _expect(qp, L.qgemm_a8w4_blockq_f32(C.c_void_p(FAKE), 2, 128, 128, C.byref(i4),
                                        C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 64,
                                        C.c_void_p(FAKE * 16), 1 << 20, None),
            qp.QP_EUNSUPPORTED, "asymmetric")
    i4.format = 2
    _expect(qp, L.qgemm_a8w8_blockwise_f32(C.c_void_p(FAKE), 2, 128, 128, C.byref(i4),
                                           C.c_void_p(FAKE), None, -6.0, 6.0, C.c_void_p(FAKE), 64,
                                           C.c_void_p(FAKE * 16), 1 << 20, None),
            qp.QP_EINVAL, "block-quantized")
    # unpack: channel range outside the blob; zero points of an int4 blob
    _expect(qp, L.qunpack_weights(C.byref(i8), C.c_void_p(FAKE), 60, 20, C.c_void_p(FAKE), 129,
                                  None, 0, None, None, 0, None), qp.QP_EINVAL, "outside")
    _expect(qp, L.qunpack_weights(C.byref(i4), C.c_void_p(FAKE), 0, 4, None, 0, None, 0,
                                  C.c_void_p(FAKE), None, 0, None), qp.QP_EINVAL, "zero points")


def test_conv_routes_and_workspace(qp):
    """qconv2d_s8 picks the 1x1 fastway (GEMM workspace), the implicit GEMM
    (no workspace) for C % 16 == 0, and the explicit im2col otherwise; bad
    dilation is refused."""
    L = qp.lib()
    n = C.c_size_t()

    def ws(C_, KH, pads, dil=(1, 1), stride=(1, 1)):
        x = qp.qtensor(qp.QP_S8, [2, 8, 8, C_], [64 * C_, 8 * C_, C_, 1], scale=0.05)
        info = _info8(qp, N=40, K=KH * KH * C_)
        st = L.qconv2d_s8_ws_size(C.byref(x), C.byref(info), KH, KH, stride[0], stride[1], *pads,
                                  dil[0], dil[1], C.byref(n))
        return st, n.value

    assert ws(64, 1, (0, 0, 0, 0)) == (qp.QP_OK, 128 * 64)          # fastway: GEMM copy of x
    assert ws(32, 3, (1, 1, 1, 1)) == (qp.QP_OK, 0)                 # implicit
    assert ws(16, 3, (2, 2, 2, 2), (2, 2)) == (qp.QP_OK, 0)
    st, b = ws(3, 3, (1, 1, 1, 1))                                  # explicit im2col
    assert st == qp.QP_OK and b >= 128 * 64
    assert ws(16, 3, (1, 1, 1, 1), (0, 1))[0] == qp.QP_EINVAL
    assert ws(16, 3, (0, 0, 0, 0), (4, 4))[0] == qp.QP_EINVAL       # span 9 > 8


def test_repack_checks_the_buffer_before_any_launch(qp):
    """qrepack_weights refuses weights whose blob geometry differs from the
    buffer's description (host-side check; nothing is launched)."""
    L = qp.lib()
    i8 = _info8(qp)                                  # int8, N=70, K=129
    for N, K in [(70, 130), (71, 129)]:
        d = _w8_desc(qp, N, K, scheme=qp.QP_PER_CHANNEL)
        _expect(qp, L.qrepack_weights(C.byref(d), C.c_void_p(FAKE), 1, 0, C.c_void_p(FAKE),
                                      C.byref(i8), None), qp.QP_EINVAL,
                "qrepack_weights: the buffer holds")
    d4 = qp.qtensor(qp.QP_S4, [70, 129], [129, 1], scheme=qp.QP_BLOCKWISE, group_size=32)
    _expect(qp, L.qrepack_weights(C.byref(d4), C.c_void_p(FAKE), 1, 0, C.c_void_p(FAKE),
                                  C.byref(i8), None), qp.QP_EINVAL, "format 1")
    _expect(qp, L.qrepack_weights(C.byref(d4), C.c_void_p(FAKE), 1, 0, C.c_void_p(FAKE),
                                  None, None), qp.QP_EINVAL, "null argument")
    assert i8.N == 70 and i8.K == 129 and i8.format == 1   # untouched
