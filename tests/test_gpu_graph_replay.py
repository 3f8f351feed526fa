"""The hot-path entry points inside a captured HIP graph: every replay, with
eager work and synchronizations in between (the outputs are cleared
eagerly before each replay), must reproduce the eager call's output
bit for bit.  Nothing on these paths allocates, memsets or synchronizes,
so each call is one or two plain kernel launches on the caller's stream."""
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


def _replays_match(call, out, replays=3):
    import torch
    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(replays):
        out.zero_()                       # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d differs from the eager call" % r
    del g


def test_graph_int8_gemm_and_conv(qp):
    import torch
    print("graph: int8 GEMM 130x70x129, implicit conv 56x56x64", flush=True)
    g = synth.gemm_affine_per_tensor()
    blob, info = qp.pack_s8(_dev(g["B"]), scale=g["sB"], zero_point=g["zB"], k_axis=0, n_axis=1)
    A, bias = _dev(g["A"]), _dev(g["bias"])
    a_desc = qp.qtensor(qp.QP_S8, list(A.shape), [A.stride(0), 1], scale=g["sA"],
                        zero_point=g["zA"])
    ws = torch.empty(max(qp.qgemm_s8s8_requant_ws_size(a_desc, info), 256), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((A.shape[0], info.N), dtype=torch.int8, device="cuda")
    _replays_match(lambda: qp.qgemm_s8s8_requant(A, g["sA"], g["zA"], blob, info, bias, 1000,
                                                 g["s_out"], g["zp_out"], g["relu"], out=out,
                                                 ws=ws), out)
    c = synth.conv3x3_nhwc()
    bc, ic = qp.pack_s8(_dev(c["W"]), scales=_dev(c["s_w"]))
    X, bc_bias = _dev(c["X"]), _dev(c["bias"])
    yc = torch.empty((1, 56, 56, 64), dtype=torch.int8, device="cuda")
    wsc = torch.empty(256, dtype=torch.uint8, device="cuda")
    _replays_match(lambda: qp.qconv2d_s8(X, c["s_in"], c["zp_in"], bc, ic, 3, 3, c["stride"],
                                         c["pad"], (1, 1), bc_bias, 1000, c["s_out"], c["zp_out"],
                                         True, out=yc, ws=wsc), yc)


@pytest.mark.parametrize("M", [1, 16, 40])
def test_graph_a8w4_with_quantization(qp, M):
    import torch
    print("graph: A8W4 M=%d" % M, flush=True)
    a = synth.a8w4(synth.BASE_SEED + 31, M, 320, 1024)
    blob, info = qp.pack_s4(_dev(a["W"]), _dev(a["sw"]))
    X, bias = _dev(a["X"]), _dev(a["bias"])
    out = torch.empty((M, 320), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(qp.qgemm_a8w4_blockwise_f32_ws_size(M, info), 256), dtype=torch.uint8,
                     device="cuda")
    _replays_match(lambda: qp.qgemm_a8w4_blockwise_f32(X, blob, info, bias, -6.0, 6.0, out=out,
                                                       ws=ws), out)
    wsb = torch.empty(max(qp.qgemm_a8w4_blockq_f32_ws_size(M, info), 256), dtype=torch.uint8,
                      device="cuda")
    _replays_match(lambda: qp.qgemm_a8w4_blockq_f32(X, blob, info, bias, -6.0, 6.0, out=out,
                                                    ws=wsb), out)


def test_graph_block_quantized_int8(qp):
    import torch
    print("graph: block-quantized int8 GEMM and conv", flush=True)
    rng = np.random.default_rng(41)
    N, K, M = 200, 512, 5
    W = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(1e-4, 1e-3, (N, K // 128)).astype(np.float32)
    blob, info = qp.pack_s8_blockwise(_dev(W), _dev(sw), block=128)
    X = _dev(rng.standard_normal((M, K)).astype(np.float32))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(qp.qgemm_a8w8_blockwise_f32_ws_size(M, info), 256), dtype=torch.uint8,
                     device="cuda")
    _replays_match(lambda: qp.qgemm_a8w8_blockwise_f32(X, blob, info, None, -6.0, 6.0, out=out,
                                                       ws=ws), out)
    Wc = rng.integers(-127, 128, (48, 64, 3, 3)).astype(np.int8)
    swc = rng.uniform(1e-4, 1e-3, (48, 1)).astype(np.float32)
    bc, ic = qp.pack_s8_blockwise(_dev(Wc), _dev(swc), block=64)
    Xc = _dev(rng.integers(-128, 128, (2, 12, 12, 64)).astype(np.int8))
    yc = torch.empty((2, 12, 12, 48), dtype=torch.float32, device="cuda")
    _replays_match(lambda: qp.qconv2d_s8_blockwise_f32(Xc, 0.05, 3, bc, ic, 3, 3, (1, 1),
                                                       (1, 1, 1, 1), (1, 1), None, -6.0, 6.0,
                                                       out=yc), yc)
