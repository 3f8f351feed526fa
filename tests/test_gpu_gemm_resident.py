"""GPU parity of the small-GEMM single launch: 64x64 tiles whose activations
are read byte-exact into LDS (any row stride, any base alignment, K not a
multiple of 64) with the row sums for weight zero points formed on the way.
Bit-exact against the oracle's INT32 accumulator (O1) and requantization
(O3) for every output.  These shapes take no workspace at all: a call with
an empty one succeeds only if no A copy or row-sum pass is launched."""
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


def _first_diff(got, want, what, acc=None):
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        extra = "" if acc is None else " (oracle int32 acc %d)" % acc[i]
        raise AssertionError("%s: %d mismatches, first at %s: gpu=%s oracle=%s%s"
                             % (what, len(bad), i, got[i], want[i], extra))


def _strided_view(A, lda, offset):
    """A [M,K] placed at byte `offset` of a flat device buffer with row stride
    `lda`; the bytes around it hold a pattern the GEMM must not read."""
    import torch
    M, K = A.shape
    flat = np.full(offset + max(M - 1, 0) * lda + K + 64, 0x5A, np.uint8).view(np.int8)
    for m in range(M):
        flat[offset + m * lda: offset + m * lda + K] = A[m]
    d = _dev(flat)
    return torch.as_strided(d, (M, K), (lda, 1), offset)


def _case(qp, orc, M, N, K, lda, offset, per_channel, seed, out="s8"):
    import torch
    print("resident gemm M=%d N=%d K=%d lda=%d off=%d zp=%s" % (M, N, K, lda, offset, per_channel),
          flush=True)
    rng = np.random.default_rng(seed)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-128, 128, (K, N)).astype(np.int8)
    zA = int(rng.integers(-128, 128))
    if per_channel:
        zB = rng.integers(-30, 31, N).astype(np.int32)
        sB = rng.uniform(0.001, 0.02, N).astype(np.float32)
        blob, info = qp.pack_s8(_dev(B), scales=_dev(sB), zero_points=_dev(zB), k_axis=0,
                                n_axis=1)
    else:
        zB = np.full(N, int(rng.integers(-30, 31)), np.int32)
        sB = np.full(N, 0.01, np.float32)
        blob, info = qp.pack_s8(_dev(B), scale=0.01, zero_point=int(zB[0]), k_axis=0, n_axis=1)
    bias = rng.integers(-5000, 5001, N).astype(np.int32)
    dA = _strided_view(A, lda, offset)
    a_desc = qp.qtensor(qp.QP_S8, [M, K], [lda, 1])
    assert qp.qgemm_s8s8_requant_ws_size(a_desc, info) == 0
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    acc = orc.gemm_affine(A, zA, B, zB, bias)
    if out == "s32":
        c = qp.qgemm_s8s8_requant(dA, 0.02, zA, blob, info, _dev(bias), 5000, out_dtype="s32",
                                  ws=empty)
        _first_diff(c.cpu().numpy(), acc.astype(np.int32), "int32 accumulator")
    else:
        s_out, zp_out = float(rng.uniform(0.05, 2.0)), int(rng.integers(-128, 128))
        c = qp.qgemm_s8s8_requant(dA, 0.02, zA, blob, info, _dev(bias), 5000, s_out, zp_out,
                                  bool(seed % 2), ws=empty)
        want, _ = orc.requant_matrix(acc, 0.02, sB, s_out, zp_out, bool(seed % 2))
        _first_diff(c.cpu().numpy(), want, "int8 output", acc)


def test_worked_shape_needs_no_workspace(qp, orc):
    """The 130x70x129 per-tensor GEMM: K = 129 is two full K tiles and one
    byte, lda = 129 leaves every row but the first unaligned."""
    import torch
    d = synth.gemm_affine_per_tensor()
    blob, info = qp.pack_s8(_dev(d["B"]), scale=d["sB"], zero_point=d["zB"], k_axis=0, n_axis=1)
    a_desc = qp.qtensor(qp.QP_S8, [130, 129], [129, 1])
    assert qp.qgemm_s8s8_requant_ws_size(a_desc, info) == 0
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    got = qp.qgemm_s8s8_requant(_dev(d["A"]), d["sA"], d["zA"], blob, info, _dev(d["bias"]),
                                1000, d["s_out"], d["zp_out"], d["relu"], ws=empty)
    acc = orc.gemm_affine(d["A"], d["zA"], d["B"], d["zB"], d["bias"])
    want, _ = orc.requant_matrix(acc, d["sA"], d["sB"], d["s_out"], d["zp_out"], d["relu"])
    _first_diff(got.cpu().numpy(), want, "worked-shape int8 output", acc)


@pytest.mark.parametrize("K", [1, 3, 15, 16, 17, 63, 64, 65, 127, 129, 255, 257, 500, 959, 960])
def test_k_tails(qp, orc, K):
    _case(qp, orc, 67, 45, K, K, 0, True, K)


@pytest.mark.parametrize("lda,offset", [(131, 1), (132, 4), (136, 8), (144, 16), (129, 3),
                                        (200, 7), (4099, 2)])
def test_strides_and_base_alignment(qp, orc, lda, offset):
    _case(qp, orc, 130, 70, 129, lda, offset, lda % 2 == 0, lda + offset)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 300, 100), (64, 64, 64), (65, 65, 65),
                                   (200, 33, 300), (190, 130, 900)])
def test_ragged_tiles(qp, orc, M, N, K):
    _case(qp, orc, M, N, K, K + 5, 1, True, M * N + K)
    _case(qp, orc, M, N, K, K, 0, False, M * N + K + 1, out="s32")


def test_row_sums_at_extremes(qp, orc):
    """All-(-128) activations over the deepest resident K with weight zero
    points: the row sums reach -122880 and must cancel exactly."""
    import torch
    K, M, N = 960, 70, 40
    A = np.full((M, K), -128, np.int8)
    A[1::2] = 127
    B = np.full((K, N), 127, np.int8)
    zB = np.arange(N, dtype=np.int32) - 20
    blob, info = qp.pack_s8(_dev(B), scales=_dev(np.full(N, 1e-6, np.float32)),
                            zero_points=_dev(zB), k_axis=0, n_axis=1)
    got = qp.qgemm_s8s8_requant(_dev(A[:, :]), 1.0, 0, blob, info, out_dtype="s32",
                                ws=torch.empty(0, dtype=torch.uint8, device="cuda"))
    acc = orc.gemm_affine(A, 0, B, zB)
    _first_diff(got.cpu().numpy(), acc.astype(np.int32), "extreme row sums")


def test_deeper_k_keeps_workspace_plan(qp, orc):
    """K = 961 exceeds what the resident kernel holds: the copy plan with a
    workspace is used, and its result is the same exact accumulator."""
    rng = np.random.default_rng(961)
    M, N, K = 50, 30, 961
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    B = rng.integers(-128, 128, (K, N)).astype(np.int8)
    zB = rng.integers(-10, 11, N).astype(np.int32)
    blob, info = qp.pack_s8(_dev(B), scales=_dev(np.full(N, 0.01, np.float32)),
                            zero_points=_dev(zB), k_axis=0, n_axis=1)
    assert qp.qgemm_s8s8_requant_ws_size(qp.qtensor(qp.QP_S8, [M, K], [K, 1]), info) > 0
    got = qp.qgemm_s8s8_requant(_dev(A), 0.02, 5, blob, info, out_dtype="s32")
    _first_diff(got.cpu().numpy(), orc.gemm_affine(A, 5, B, zB).astype(np.int32),
                "K=961 accumulator")
