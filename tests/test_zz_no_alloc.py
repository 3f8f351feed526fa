"""qgemm_a8w4_blockwise_f32_noalloc (no workspace argument; the library's
per-GPU scratch array holds the quantized rows) against
qgemm_a8w4_blockwise_f32 with a caller workspace: the same kernels, so the
outputs must be identical, and both within 1e-5*max(1,|o|) of the oracle.
Two calls in a row, the second with fewer rows, so the second runs on the
scratch contents the first left behind; the one-row call, which needs no
scratch; and the size limit, refused on the host."""
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


def _within(got, want):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    return bool((err <= 1e-5 * np.maximum(1.0, np.abs(want.astype(np.float64)))).all())


def test_noalloc_matches_workspace_entry_point(qp, orc):
    import torch
    d = synth.a8w4_gemm(128)                       # M=128, K=4096, N=11008
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    bias = _dev(d["bias"])
    rng = np.random.default_rng(5)
    X2 = rng.standard_normal((16, 4096)).astype(np.float32)
    for X in (d["X"], X2):                         # the second call: fewer rows
        print("no-alloc A8W4, M =", X.shape[0], flush=True)
        dX = _dev(X)
        got = qp.qgemm_a8w4_blockwise_f32_noalloc(dX, blob, info, bias, -6.0, 6.0)
        want = qp.qgemm_a8w4_blockwise_f32(dX, blob, info, bias, -6.0, 6.0)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "no-alloc output differs from the workspace entry point"
        oracle = orc.rows_in_threads(orc.a8w4_forward, X, d["W"], d["sw"], d["bias"], -6.0, 6.0)
        assert _within(got.cpu().numpy(), oracle)


def test_noalloc_single_row_and_limit(qp, orc):
    import torch
    d = synth.a8w4_gemv()                          # M=1, K=N=4096: no scratch used
    blob, info = qp.pack_s4(_dev(d["W"]), _dev(d["sw"]))
    dX = _dev(d["X"])
    got = qp.qgemm_a8w4_blockwise_f32_noalloc(dX, blob, info, _dev(d["bias"]), -6.0, 6.0)
    want = qp.qgemm_a8w4_blockwise_f32(dX, blob, info, _dev(d["bias"]), -6.0, 6.0)
    assert torch.equal(got, want)
    # 1024 rows of K = 4096 need 4 MiB + 8 KiB of scratch: refused, nothing launched
    big = torch.zeros((1024, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(qp.QPackError) as e:
        qp.qgemm_a8w4_blockwise_f32_noalloc(big, blob, info)
    assert e.value.status == qp.QP_ESIZE
    # 1022 rows fill the 4 MiB exactly and still agree
    X = np.random.default_rng(6).standard_normal((1022, 4096)).astype(np.float32)
    dX = _dev(X)
    got = qp.qgemm_a8w4_blockwise_f32_noalloc(dX, blob, info)
    want = qp.qgemm_a8w4_blockwise_f32(dX, blob, info)
    assert torch.equal(got, want)
