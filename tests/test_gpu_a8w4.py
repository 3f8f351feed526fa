"""GPU parity of the A8W4 blockwise path (dynamic row quantization, int4
group-32 weights, f32 dequantize + bias + clamp) against the oracle:
|gpu - oracle| <= 1e-5 * max(1, |oracle|) for every output."""
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
    return float((err / np.maximum(1.0, np.abs(want))).max())


def _case(qp, orc, d, rows=None):
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    Y = _host(qp.qgemm_a8w4_blockwise_f32(_dev(d["X"]), blob, info, _dev(d["bias"]),
                                          d["clamp_lo"], d["clamp_hi"]))
    X = d["X"] if rows is None else d["X"][rows]
    want = orc.rows_in_threads(orc.a8w4_forward, X, d["W"], d["sw"], d["bias"], d["clamp_lo"],
                               d["clamp_hi"])
    got = Y if rows is None else Y[rows]
    return _check_close(got, want, "a8w4 f32 output")


def test_a8w4_gemv_workload(qp, orc):
    _case(qp, orc, synth.a8w4_gemv())


@pytest.mark.parametrize("M", [16, 128])
def test_a8w4_gemm_workload(qp, orc, M):
    _case(qp, orc, synth.a8w4_gemm(M))


@pytest.mark.parametrize("M,N,K", [(1, 70, 96), (1, 1, 32), (2, 130, 200), (3, 64, 4096),
                                   (5, 77, 1000), (17, 100, 256), (40, 33, 64), (1, 4096, 33),
                                   (33, 48, 160), (65, 40, 256), (130, 48, 320),
                                   (1, 40, 32768), (1, 37, 40000), (7, 50, 1500),
                                   (16, 64, 2048), (12, 200, 3000), (4, 40, 5000),
                                   (48, 96, 512), (100, 33, 1536), (128, 64, 1024),
                                   # K exactly four ranges of eight blocks at a ragged N;
                                   # grids whose workgroups are placed by XCD (row groups
                                   # of a channel group together), exact and ragged K
                                   (16, 40, 4096), (60, 250, 512), (100, 330, 512),
                                   (100, 250, 640),
                                   # 513..768 channel tiles: three tiles a workgroup at
                                   # M <= 16, the grid's last waves on a repeated tile
                                   (5, 8300, 1000), (16, 9050, 4096), (2, 12280, 384)])
def test_a8w4_small_shapes_and_tails(qp, orc, M, N, K):
    _case(qp, orc, synth.a8w4(synth.BASE_SEED + 7 * M + N + K, M, N, K))


def test_a8w4_prequantized_entry(qp, orc):
    d = synth.a8w4(synth.BASE_SEED + 50, 3, 300, 512)
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    import torch
    q = torch.zeros((3, info.Kpad), dtype=torch.int8, device="cuda")
    q, s, z = qp.qquantize_rows_s8(_dev(d["X"]), q=q)
    Y = _host(qp.qgemm_a8w4_prequant_f32(q, s, z, blob, info, _dev(d["bias"]), -6.0, 6.0))
    want = orc.a8w4_forward(d["X"], d["W"], d["sw"], d["bias"], -6, 6)
    _check_close(Y, want, "prequant a8w4")


def test_a8w4_no_bias_no_clamp(qp, orc):
    d = synth.a8w4(synth.BASE_SEED + 60, 1, 256, 512)
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    Y = _host(qp.qgemm_a8w4_blockwise_f32(_dev(d["X"]), blob, info))
    want = orc.a8w4_forward(d["X"], d["W"], d["sw"], None, -3.4e38, 3.4e38)
    _check_close(Y, want, "a8w4 without bias or clamp")


def test_a8w4_deterministic(qp):
    d = synth.a8w4_gemv()
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    X, b = _dev(d["X"]), _dev(d["bias"])
    first = _host(qp.qgemm_a8w4_blockwise_f32(X, blob, info, b, -6.0, 6.0))
    for _ in range(10):
        assert np.array_equal(first, _host(qp.qgemm_a8w4_blockwise_f32(X, blob, info, b, -6.0, 6.0)))


# ---- group scales stored as bf16 (blob format 3): the oracle takes the
# scales rounded by O6b, everything else unchanged
def _case_bf16(qp, orc, d, rows=None, prequant=False):
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]), scale_dtype="bf16")
    assert info.format == 3
    sw16 = orc.round_bf16(d["sw"])
    if prequant:
        import torch
        M = d["X"].shape[0]
        q = torch.zeros((M, info.Kpad), dtype=torch.int8, device="cuda")
        q, s, z = qp.qquantize_rows_s8(_dev(d["X"]), q=q)
        Y = _host(qp.qgemm_a8w4_prequant_f32(q, s, z, blob, info, _dev(d["bias"]),
                                             d["clamp_lo"], d["clamp_hi"]))
    else:
        Y = _host(qp.qgemm_a8w4_blockwise_f32(_dev(d["X"]), blob, info, _dev(d["bias"]),
                                              d["clamp_lo"], d["clamp_hi"]))
    X = d["X"] if rows is None else d["X"][rows]
    want = orc.rows_in_threads(orc.a8w4_forward, X, d["W"], sw16, d["bias"], d["clamp_lo"],
                               d["clamp_hi"])
    _check_close(Y if rows is None else Y[rows], want, "a8w4 bf16-scale output")
    return blob, info, sw16


def test_a8w4_bf16_scales_gemv_workload(qp, orc):
    d = synth.a8w4_gemv()
    blob, info, sw16 = _case_bf16(qp, orc, d)
    # the blob holds exactly the rounded scales, and they differ from the f32 ones
    _, sc, _, _ = qp.qunpack_weights(blob, info, values=False)
    assert np.array_equal(_host(sc), sw16) and not np.array_equal(sw16, d["sw"])


@pytest.mark.parametrize("M", [16, 128])
def test_a8w4_bf16_scales_gemm_workload(qp, orc, M):
    _case_bf16(qp, orc, synth.a8w4_gemm(M))


@pytest.mark.parametrize("M,N,K,prequant", [(1, 70, 96, False), (3, 64, 4096, True),
                                            (5, 77, 1000, False), (33, 48, 160, True),
                                            (130, 48, 320, False), (9, 40, 1800, True),
                                            (14, 33, 2500, False), (64, 40, 1024, False),
                                            (33, 70, 512, True), (60, 250, 512, True),
                                            (100, 250, 640, False)])
def test_a8w4_bf16_scales_shapes(qp, orc, M, N, K, prequant):
    _case_bf16(qp, orc, synth.a8w4(synth.BASE_SEED + 11 * M + N + K, M, N, K), prequant=prequant)


# ---- asymmetric int4 (blob format 4): a float offset per group, oracle O6c
def _offsets(d, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-0.05, 0.05, d["sw"].shape).astype(np.float32)


def _case_asym(qp, orc, d, bw, rows=None, prequant=False):
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]), offsets=_dev(bw))
    assert info.format == 4
    if prequant:
        import torch
        M = d["X"].shape[0]
        q = torch.zeros((M, info.Kpad), dtype=torch.int8, device="cuda")
        q, s, z = qp.qquantize_rows_s8(_dev(d["X"]), q=q)
        Y = _host(qp.qgemm_a8w4_prequant_f32(q, s, z, blob, info, _dev(d["bias"]),
                                             d["clamp_lo"], d["clamp_hi"]))
    else:
        Y = _host(qp.qgemm_a8w4_blockwise_f32(_dev(d["X"]), blob, info, _dev(d["bias"]),
                                              d["clamp_lo"], d["clamp_hi"]))
    X = d["X"] if rows is None else d["X"][rows]
    want = orc.rows_in_threads(orc.a8w4_forward_asym, X, d["W"], d["sw"], bw, d["bias"],
                               d["clamp_lo"], d["clamp_hi"])
    _check_close(Y if rows is None else Y[rows], want, "asymmetric a8w4 output")
    return blob, info


def test_a8w4_asym_gemv_workload(qp, orc):
    d = synth.a8w4_gemv()
    bw = _offsets(d, 1)
    blob, info = _case_asym(qp, orc, d, bw)
    _, sc, _, dq = qp.qunpack_weights(blob, info, values=False, dequant=True)
    pairs = _host(sc).reshape(4096, -1, 2)
    assert np.array_equal(pairs[..., 0], bw) and np.array_equal(pairs[..., 1], d["sw"])
    assert np.array_equal(_host(dq), orc.dequant_weights_s4(d["W"], d["sw"], 32, bw))


@pytest.mark.parametrize("M", [16, 128])
def test_a8w4_asym_gemm_workload(qp, orc, M):
    d = synth.a8w4_gemm(M)
    _case_asym(qp, orc, d, _offsets(d, M))


@pytest.mark.parametrize("M,N,K,prequant", [(1, 70, 96, False), (1, 33, 1000, False),
                                            (3, 64, 4096, True), (5, 77, 1000, False),
                                            (33, 48, 160, True), (40, 33, 64, False),
                                            (130, 48, 320, False), (9, 40, 1800, True),
                                            (14, 33, 2500, False), (64, 40, 1024, False),
                                            (33, 70, 512, True), (100, 330, 512, False),
                                            (16, 40, 4096, True)])
def test_a8w4_asym_shapes(qp, orc, M, N, K, prequant):
    d = synth.a8w4(synth.BASE_SEED + 13 * M + N + K, M, N, K)
    _case_asym(qp, orc, d, _offsets(d, M + N + K), prequant=prequant)


# ---- activations quantized per block of 32 (O5b), product O6d
@pytest.mark.parametrize("M,K", [(1, 4096), (3, 100), (130, 320), (16, 4096), (5, 33)])
def test_quantize_rows_blocked_bit_exact(qp, orc, M, K):
    rng = np.random.default_rng(M * 7 + K)
    X = (rng.standard_normal((M, K)) * rng.uniform(0.05, 20, (M, 1))).astype(np.float32)
    if K >= 64:
        X[0, 32:64] = 0.0                          # an all-zero block
        X[-1, :32] = np.abs(X[-1, :32]) + 0.5      # an all-positive block
    kpad = ((K + 127) // 128) * 128
    q, sc, zp = qp.qquantize_rows_s8_blocked(_dev(X), kpad=kpad)
    q, sc, zp = _host(q), _host(sc), _host(zp)
    wq, ws, wz = orc.quantize_rows_s8_blocked(X, 32)
    G = (K + 31) // 32
    assert np.array_equal(q[:, :K], wq) and not q[:, K:].any()
    assert np.array_equal(sc[:, :G], ws) and np.array_equal(zp[:, :G], wz)
    assert np.all(sc[:, G:] == 1.0) and not zp[:, G:].any()


def _case_bq(qp, orc, d, rows=None, prequant=False, scale_dtype="f32"):
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]), scale_dtype=scale_dtype)
    sw = orc.round_bf16(d["sw"]) if scale_dtype == "bf16" else d["sw"]
    if prequant:
        q, sa, za = qp.qquantize_rows_s8_blocked(_dev(d["X"]), kpad=info.Kpad)
        Y = _host(qp.qgemm_a8w4_blockq_prequant_f32(q, sa, za, blob, info, _dev(d["bias"]),
                                                    d["clamp_lo"], d["clamp_hi"]))
    else:
        Y = _host(qp.qgemm_a8w4_blockq_f32(_dev(d["X"]), blob, info, _dev(d["bias"]),
                                           d["clamp_lo"], d["clamp_hi"]))
    X = d["X"] if rows is None else d["X"][rows]
    want = orc.rows_in_threads(orc.a8w4_forward_blockq, X, d["W"], sw, d["bias"], d["clamp_lo"],
                               d["clamp_hi"])
    _check_close(Y if rows is None else Y[rows], want, "per-block a8w4 output")


def test_a8w4_blockq_gemv_workload(qp, orc):
    _case_bq(qp, orc, synth.a8w4_gemv())


@pytest.mark.parametrize("M", [16, 128])
def test_a8w4_blockq_gemm_workload(qp, orc, M):
    _case_bq(qp, orc, synth.a8w4_gemm(M))


@pytest.mark.parametrize("M,N,K,prequant,sdt", [(1, 70, 96, False, "f32"),
                                                (1, 33, 1000, True, "bf16"),
                                                (1, 40, 1000, False, "bf16"),
                                                (1, 16, 53248, False, "f32"),
                                                (1, 48, 32768, False, "f32"),
                                                (1, 50, 20000, False, "bf16"),
                                                (2, 130, 200, False, "f32"),
                                                (5, 77, 1000, True, "f32"),
                                                (17, 100, 256, False, "bf16"),
                                                (33, 48, 160, True, "f32"),
                                                (130, 48, 320, False, "f32"),
                                                (3, 40, 2048, False, "bf16"),
                                                (16, 70, 2100, True, "f32"),
                                                (18, 100, 1000, False, "bf16"),
                                                (40, 64, 40000, False, "f32"),
                                                (97, 130, 2048, True, "f32")])
def test_a8w4_blockq_shapes(qp, orc, M, N, K, prequant, sdt):
    _case_bq(qp, orc, synth.a8w4(synth.BASE_SEED + 17 * M + N + K, M, N, K), prequant=prequant,
             scale_dtype=sdt)


def test_a8w4_blockq_gemv_unaligned_row(qp, orc):
    """One row quantized per block inside the GEMV (no workspace), read
    from 4 bytes past a 16-byte boundary."""
    import torch
    d = synth.a8w4(synth.BASE_SEED + 95, 1, 70, 900)
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    assert qp.qgemm_a8w4_blockq_f32_ws_size(1, info) == 0
    big = torch.zeros((1, 904), dtype=torch.float32, device="cuda")
    big[:, 1:901] = _dev(d["X"])
    Xv = big[:, 1:901]
    assert Xv.data_ptr() % 16 == 4
    Y = _host(qp.qgemm_a8w4_blockq_f32(Xv, blob, info, _dev(d["bias"]), d["clamp_lo"],
                                       d["clamp_hi"]))
    want = orc.a8w4_forward_blockq(d["X"], d["W"], d["sw"], d["bias"], d["clamp_lo"],
                                   d["clamp_hi"])
    _check_close(Y, want, "per-block a8w4 GEMV, unaligned row")


def test_a8w4_blockq_rejects_asymmetric_weights(qp):
    d = synth.a8w4(synth.BASE_SEED + 90, 2, 32, 64)
    bw = np.zeros_like(d["sw"])
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]), offsets=_dev(bw))
    with pytest.raises(qp.QPackError):
        qp.qgemm_a8w4_blockq_f32(_dev(d["X"]), blob, info)
