"""GPU proof of the requantizing epilogue's own edge cases, bit-exact against
oracle O3 ("Quantized GEMM: numeric contract, SRAM, DMA and result
verification", section 1: ONNX QuantizeLinear rounding -- half to even --
and saturation, with the integer multiplier/shift realisation; MNN
"ConvInt8TiledExecutor.cpp": with ReLU the lower clamp is the output zero
point).

Every launch uses per-channel weight scales with sA = sOut = 1, so column n
has the multiplier M_n = sB[n] and the launch covers many multipliers at
once:
  * exact ties: M_n = c * 2^-s with c in {1, 3/4, 5/8}.  acc * M_n is j + 1/2
    exactly when the 2-adic valuation of acc is s-1, s+1 or s+2.  Weights and
    bias of column n are multiples of 2^b with b that valuation, so about
    half of the column's accumulators are exact ties (the test counts them in
    integers and requires many, rounding both up and down);
  * all multipliers in [2^-23, 1/2) select the epilogue that rounds in
    32-bit pieces (shifts 32..53) from one folded 64-bit addend per column;
    one multiplier of 1/2 or more (shift 21 for 1000, 29 for 3, 31 for 1/2
    and 3/4), or one below 2^-23, selects the 64-bit one;
  * M = 2^-70 (shift >= 63: every output is the output zero point) and
    M = 2^30 (shift 0: every non-zero accumulator saturates);
  * ReLU with a non-zero output zero point; M = 2^31 (shift < 0) is refused.
The GEMM is checked through qgemm_s8s8_requant; the convolution through
qconv2d_s8 (implicit GEMM, and the explicit route for C % 16 != 0) and
qconv2d_s8_im2col."""
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


def _host(t):
    return t.cpu().numpy()


# (c, s, b): multiplier c * 2^-s; b = the valuation of acc that makes a tie
_TIES_HI = ([(1.0, s, s - 1) for s in range(2, 9)] + [(0.75, s, s + 1) for s in range(1, 7)] +
            [(0.625, s, s + 2) for s in range(1, 6)])
# no ties possible or wanted: shifts 32..61 away from the tie columns, and
# M = 2^-70 (shift >= 63); multipliers below 2^-23 (shifts above 53) move a
# launch whose multipliers are all below 1/2 from the 32-bit-piece rounding
# with the folded 64-bit addend to the general 64-bit rounding
_WIDE_HI = [(1.0, 12, 0), (1.0, 20, 0), (1.0, 30, 0), (0.75, 25, 0), (1.0, 70, 0)]
# the same without the multipliers below 2^-23 (shifts up to 53: 0.75 * 2^-22
# has shift 53), so the launch keeps the 32-bit-piece rounding
_FOLD_HI = [(1.0, 12, 0), (1.0, 20, 0), (1.0, 22, 0), (0.75, 22, 0)]
# columns that force the 64-bit rounding (multiplier >= 1/2), plus the
# shift >= 63 and shift == 0 mappings
_LO_ONLY = [(1.0, 1, 0), (0.75, 0, 1), (3.0, 0, 0), (1000.0, 0, 0), (1.0, -30, 0), (1.0, 70, 0)]


def _columns(spec):
    mult = np.array([np.float32(c * 2.0 ** -s) for c, s, _ in spec], np.float32)
    val = np.array([b for _, _, b in spec], np.int64)
    return mult, val


def _operand_cols(rng, K, val):
    """[K, N] int8 weights: column n is 2^val[n] times a sparse {-1, 0, 1}
    pattern (only -1 when 2^val[n] = 128)."""
    N = val.size
    Bp = np.zeros((K, N), np.int64)
    for n in range(N):
        idx = rng.choice(K, size=min(K, 5), replace=False)
        Bp[idx, n] = rng.choice([-1, 1], size=idx.size)
        if val[n] >= 7:
            Bp[:, n] = -np.abs(Bp[:, n])
    B = Bp << val[None, :]
    assert B.min() >= -128 and B.max() <= 127
    return B.astype(np.int8)


def _bias_cols(rng, val):
    return (rng.integers(-3, 4, val.size).astype(np.int64) << val).astype(np.int32)


def _tie_stats(orc, acc, mult):
    """(exact ties, ties inside the int8 range with an even floor, with an odd
    floor) over all outputs, in exact integer arithmetic."""
    ties = even = odd = 0
    for n in range(acc.shape[1]):
        m0, sh = orc.requant_params(float(mult[n]))
        if not 1 <= sh <= 62:
            continue
        t = acc[:, n].astype(np.int64) * np.int64(m0)
        d = np.int64(1) << np.int64(sh)
        rem = np.mod(t, d)
        fl = np.floor_divide(t, d)
        tie = rem == (d >> np.int64(1))
        ties += int(tie.sum())
        inside = tie & (fl > -120) & (fl < 120)
        even += int((inside & (fl % 2 == 0)).sum())
        odd += int((inside & (fl % 2 == 1)).sum())
    return ties, even, odd


def _check(got, want, what, acc):
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s: gpu=%d oracle=%d (acc %d)"
                             % (what, len(bad), i, got[i], want[i], acc[i]))


def _gemm(qp, orc, A, zA, B_kn, mult, bias, zp_out, relu):
    N = B_kn.shape[1]
    blob, info = qp.pack_s8(_dev(B_kn), scales=_dev(mult), k_axis=0, n_axis=1)
    mab = int(np.abs(bias).max())
    dA = _dev(A)
    c8 = _host(qp.qgemm_s8s8_requant(dA, 1.0, zA, blob, info, _dev(bias), mab, 1.0, zp_out, relu))
    c32 = _host(qp.qgemm_s8s8_requant(dA, 1.0, zA, blob, info, _dev(bias), mab, out_dtype="s32"))
    acc = orc.gemm_affine(A, zA, B_kn, np.zeros(N, np.int32), bias)
    want, _ = orc.requant_matrix(acc, 1.0, mult, 1.0, zp_out, relu)
    _check(c32, acc.astype(np.int32), "int32 accumulator", acc)
    _check(c8, want, "int8 output", acc)
    return acc


def _activations(rng, M, K):
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    A[M // 2:] = rng.integers(-9, 10, (M - M // 2, K))   # rows whose results rarely saturate
    return A


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("zp_out,relu", [(0, False), (-2, False), (5, True), (-7, True),
                                         (127, False), (-128, False)])
def test_gemm_ties_shift_ge_32(qp, orc, zp_out, relu, wide):
    """All multipliers < 1/2: with every multiplier at least 2^-23 the
    epilogue that rounds in 32-bit pieces from one folded 64-bit addend per
    column (zero-point terms, half, output zero point); with smaller ones in
    the launch (wide) the general 64-bit rounding."""
    print("requant ties, shift >= 32, zp_out", zp_out, "relu", relu, "wide", wide, flush=True)
    rng = np.random.default_rng((40 + zp_out) % 997 + 1000 * wide)
    mult, val = _columns(_TIES_HI * 3 + (_WIDE_HI if wide else _FOLD_HI))
    M, K = 200, 128
    A = _activations(rng, M, K)
    B = _operand_cols(rng, K, val)
    acc = _gemm(qp, orc, A, 3, B, mult, _bias_cols(rng, val), zp_out, relu)
    ties, even, odd = _tie_stats(orc, acc, mult)
    assert ties >= 2000 and even >= 300 and odd >= 300, (ties, even, odd)


@pytest.mark.parametrize("zp_out,relu", [(0, False), (4, True), (-9, True)])
def test_gemm_ties_and_edges_64bit_rounding(qp, orc, zp_out, relu):
    """One multiplier >= 1/2 selects the 64-bit rounding for every column;
    the launch also holds the shift >= 63 and shift == 0 mappings."""
    print("requant ties, 64-bit rounding, zp_out", zp_out, "relu", relu, flush=True)
    rng = np.random.default_rng(70 + zp_out)
    mult, val = _columns(_LO_ONLY + _TIES_HI * 2 + _WIDE_HI)
    M, K = 150, 96                       # K != Kpad: the padded-activation path
    A = _activations(rng, M, K)
    B = _operand_cols(rng, K, val)
    acc = _gemm(qp, orc, A, -4, B, mult, _bias_cols(rng, val), zp_out, relu)
    ties, even, odd = _tie_stats(orc, acc, mult)
    assert ties >= 1000 and even >= 150 and odd >= 150, (ties, even, odd)
    # the mapped columns: 2^-70 gives the zero point, 2^30 saturates
    c70 = [i for i, (c, s, _) in enumerate(_LO_ONLY) if s == 70][0]
    c30 = [i for i, (c, s, _) in enumerate(_LO_ONLY) if s == -30][0]
    assert (acc[:, c70] != 0).any() and (acc[:, c30] != 0).any()


@pytest.mark.parametrize("wide", [False, True])
def test_gemm_large_tiles_ties(qp, orc, wide):
    """The same tie columns in the 256x256 tile configuration the large GEMM
    uses (>= 256 tiles of 256x256, K a multiple of 128): the folded-addend
    rounding in 32-bit pieces, and (wide) the general 64-bit one."""
    print("requant ties, 256x256 tiles, wide", wide, flush=True)
    rng = np.random.default_rng(91)
    base, bval = _columns(_TIES_HI + (_WIDE_HI if wide else _FOLD_HI))
    reps = 4096 // base.size + 1
    mult, val = np.tile(base, reps)[:4096], np.tile(bval, reps)[:4096]
    M, K = 4096, 256
    A = _activations(rng, M, K)
    B = _operand_cols(rng, K, val)
    bias = _bias_cols(rng, val)
    blob, info = qp.pack_s8(_dev(B), scales=_dev(mult), k_axis=0, n_axis=1)
    c8 = _host(qp.qgemm_s8s8_requant(_dev(A), 1.0, 0, blob, info, _dev(bias),
                                     int(np.abs(bias).max()), 1.0, 1, False))
    from oracle.matmul_f64 import gemm_affine_f64
    acc = gemm_affine_f64(A, 0, np.ascontiguousarray(B.T), 0, bias)
    want, _ = orc.requant_matrix(acc, 1.0, mult, 1.0, 1, False)
    _check(c8, want, "int8 output, 256x256 tiles", acc)
    ties, even, odd = _tie_stats(orc, acc[:512], mult)
    assert ties >= 20000 and even >= 3000 and odd >= 3000, (ties, even, odd)


def test_gemm_refuses_negative_shift(qp):
    import torch
    blob, info = qp.pack_s8(torch.ones((8, 64), dtype=torch.int8, device="cuda"),
                            scales=torch.full((8,), 2.0 ** 31, device="cuda"))
    A = torch.ones((4, 64), dtype=torch.int8, device="cuda")
    with pytest.raises(qp.QPackError):
        qp.qgemm_s8s8_requant(A, 1.0, 0, blob, info)
    # a restored blob refuses it the same way
    blob2, info2 = qp.blob_from_bytes(qp.blob_to_bytes(blob))
    assert (info2.scale_min, info2.scale_max) == (info.scale_min, info.scale_max)
    with pytest.raises(qp.QPackError):
        qp.qgemm_s8s8_requant(A, 1.0, 0, blob2, info2)


# ------------------------------------------------------------------ conv
def _conv_weights(rng, OC, C, KH, KW, val):
    Wp = np.zeros((OC, C * KH * KW), np.int64)
    for n in range(OC):
        idx = rng.choice(Wp.shape[1], size=4, replace=False)
        Wp[n, idx] = rng.choice([-1, 1], size=4)
        if val[n] >= 7:
            Wp[n] = -np.abs(Wp[n])
    Wt = (Wp << val[:, None]).reshape(OC, C, KH, KW)
    assert Wt.min() >= -128 and Wt.max() <= 127
    return Wt.astype(np.int8)


@pytest.mark.parametrize("route,C,spec", [
    ("implicit", 16, "hi"), ("implicit", 32, "lo"), ("explicit", 8, "hi"), ("explicit", 8, "lo"),
    ("im2col", 16, "hi"), ("im2col", 24, "lo")])
def test_conv_ties_and_edges(qp, orc, route, C, spec):
    print("requant conv", route, C, spec, flush=True)
    rng = np.random.default_rng(C * 7 + len(spec))
    mult, val = _columns(_TIES_HI + _WIDE_HI if spec == "hi" else _LO_ONLY + _TIES_HI)
    OC = mult.size
    X = rng.integers(-128, 128, (2, 11, 13, C)).astype(np.int8)
    Wt = _conv_weights(rng, OC, C, 3, 3, val)
    bias = _bias_cols(rng, val)
    blob, info = qp.pack_s8(_dev(Wt), scales=_dev(mult))
    zp_in, zp_out, relu = 7, (3 if spec == "hi" else -5), True
    mab = int(np.abs(bias).max())
    args = (_dev(X), 1.0, zp_in, blob, info, 3, 3, (1, 1), (1, 1, 1, 1))
    if route == "im2col":
        y = _host(qp.qconv2d_s8_im2col(*args, _dev(bias), mab, 1.0, zp_out, relu))
    else:
        y = _host(qp.qconv2d_s8(*args, (1, 1), _dev(bias), mab, 1.0, zp_out, relu))
    acc = orc.conv2d_direct(X, zp_in, Wt, (1, 1), (1, 1, 1, 1), bias).reshape(-1, OC)
    want, _ = orc.requant_matrix(acc, 1.0, mult, 1.0, zp_out, relu)
    _check(y.reshape(-1, OC), want, "conv int8 output (%s)" % route, acc)
    ties, even, odd = _tie_stats(orc, acc, mult)
    assert ties >= 1000 and even >= 100 and odd >= 100, (ties, even, odd)


def test_conv_refuses_negative_shift(qp):
    import torch
    blob, info = qp.pack_s8(torch.ones((8, 16, 3, 3), dtype=torch.int8, device="cuda"),
                            scales=torch.full((8,), 2.0 ** 31, device="cuda"))
    X = torch.zeros((1, 6, 6, 16), dtype=torch.int8, device="cuda")
    with pytest.raises(qp.QPackError):
        qp.qconv2d_s8(X, 1.0, 0, blob, info, 3, 3, (1, 1), (1, 1, 1, 1))
    with pytest.raises(qp.QPackError):
        qp.qconv2d_s8_im2col(X, 1.0, 0, blob, info, 3, 3, (1, 1), (1, 1, 1, 1))
