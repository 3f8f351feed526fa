"""Pins of the oracle's convolution (O4), dynamic quantizer (O5), A8W4 matmul
(O6) and packed-blob writer (O7).  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_i8(rng, shape, lo=-128, hi=127):
    return rng.integers(lo, hi + 1, size=shape).astype(np.int8)


# ------------------------------------------------------------------ O4
@pytest.mark.parametrize("case", [
    dict(NB=1, H=7, W=6, C=5, OC=4, KH=3, KW=3, stride=(1, 1), pad=(1, 1, 1, 1)),
    dict(NB=2, H=9, W=8, C=3, OC=6, KH=3, KW=2, stride=(2, 1), pad=(0, 1, 2, 0)),
    dict(NB=1, H=5, W=5, C=8, OC=3, KH=1, KW=1, stride=(1, 1), pad=(0, 0, 0, 0)),
    dict(NB=2, H=11, W=10, C=4, OC=5, KH=3, KW=3, stride=(1, 2), pad=(2, 1, 2, 3), dil=(2, 3)),
])
def test_o4_direct_equals_im2col_gemm(orc, case):
    rng = np.random.default_rng(11)
    X = _rand_i8(rng, (case["NB"], case["H"], case["W"], case["C"]))
    Wt = _rand_i8(rng, (case["OC"], case["C"], case["KH"], case["KW"]), -127, 127)
    bias = rng.integers(-1000, 1001, case["OC"]).astype(np.int32)
    zp = 7
    dil = case.get("dil", (1, 1))
    direct = orc.conv2d_direct(X, zp, Wt, case["stride"], case["pad"], bias, dil)
    col = orc.im2col(X, zp, case["KH"], case["KW"], case["stride"], case["pad"], dil)
    Bnk = Wt.transpose(0, 2, 3, 1).reshape(case["OC"], -1)   # K order (ky, kx, ic)
    acc = orc.gemm_affine(col, zp, Bnk, 0, bias, b_is_nk=True)
    assert np.array_equal(direct.reshape(-1, case["OC"]), acc)


def test_o4_pointwise_conv_is_a_plain_matmul(orc):
    rng = np.random.default_rng(12)
    X = _rand_i8(rng, (2, 4, 5, 6))
    Wt = _rand_i8(rng, (3, 6, 1, 1), -127, 127)
    out = orc.conv2d_direct(X, -4, Wt)
    want = (X.reshape(-1, 6).astype(np.int64) + 4) @ Wt[:, :, 0, 0].T.astype(np.int64)
    assert np.array_equal(out.reshape(-1, 3), want)


def test_o4_delta_kernel_closed_form(orc):
    """A weight that is 1 at the centre tap with oc == ic copies x - zp_in."""
    rng = np.random.default_rng(13)
    C = 4
    X = _rand_i8(rng, (1, 6, 7, C))
    Wt = np.zeros((C, C, 3, 3), np.int8)
    for c in range(C):
        Wt[c, c, 1, 1] = 1
    out = orc.conv2d_direct(X, 7, Wt, (1, 1), (1, 1, 1, 1))
    assert np.array_equal(out, X.astype(np.int64) - 7)
    q, _ = orc.requant_matrix(out.reshape(-1, C), 1.0, np.ones(C, np.float32), 1.0, 0, True)
    assert np.array_equal(q.reshape(out.shape), np.maximum(X.astype(np.int64) - 7, 0))


def test_o4_pad_value_only_matters_on_the_border(orc):
    rng = np.random.default_rng(14)
    X = _rand_i8(rng, (1, 8, 8, 3))
    Wt = _rand_i8(rng, (2, 3, 3, 3), -127, 127)
    zp = 7
    good = orc.im2col(X, zp, 3, 3, (1, 1), (1, 1, 1, 1))
    bad = orc.im2col(X, 0, 3, 3, (1, 1), (1, 1, 1, 1))
    Bnk = Wt.transpose(0, 2, 3, 1).reshape(2, -1)
    a_good = orc.gemm_affine(good, zp, Bnk, 0, b_is_nk=True).reshape(8, 8, 2)
    a_bad = orc.gemm_affine(bad, zp, Bnk, 0, b_is_nk=True).reshape(8, 8, 2)
    assert np.array_equal(a_good[1:-1, 1:-1], a_bad[1:-1, 1:-1])
    assert not np.array_equal(a_good[0], a_bad[0])
    assert np.array_equal(a_good, orc.conv2d_direct(X, zp, Wt, (1, 1), (1, 1, 1, 1))[0])


@pytest.mark.parametrize("dil,stride,pad", [((2, 2), (1, 1), (2, 2, 2, 2)),
                                             ((3, 1), (2, 1), (1, 0, 3, 2)),
                                             ((1, 4), (1, 3), (0, 4, 0, 4))])
def test_o4_dilation_is_a_zero_inserted_kernel(orc, dil, stride, pad):
    """A kernel dilated by d equals the undilated kernel of size d*(k-1)+1
    that holds the taps at multiples of d and zeros between (symmetric
    weights: a zero weight adds nothing, whatever the input)."""
    rng = np.random.default_rng(15)
    X = _rand_i8(rng, (2, 12, 13, 3))
    Wt = _rand_i8(rng, (4, 3, 3, 2), -127, 127)
    bias = rng.integers(-1000, 1001, 4).astype(np.int32)
    big = np.zeros((4, 3, dil[0] * 2 + 1, dil[1] * 1 + 1), np.int8)
    big[:, :, ::dil[0], ::dil[1]] = Wt
    got = orc.conv2d_direct(X, -9, Wt, stride, pad, bias, dil)
    want = orc.conv2d_direct(X, -9, big, stride, pad, bias)
    assert got.shape == want.shape and np.array_equal(got, want)
    OH, OW = orc.conv_out_dims(12, 13, 3, 2, stride, pad, dil)
    assert got.shape == (2, OH, OW, 4)


def test_o4_dilation_rejects_kernels_larger_than_the_input(orc):
    X = np.zeros((1, 4, 4, 1), np.int8)
    Wt = np.ones((1, 1, 3, 3), np.int8)
    orc.conv2d_direct(X, 0, Wt, dilation=(1, 1))
    with pytest.raises(Exception):
        orc.conv2d_direct(X, 0, Wt, dilation=(2, 2))   # spans 5 > 4 rows


# ------------------------------------------------------------------ O5
def test_o5_hand_worked_rows(orc):
    for row in _gold("dynquant_worked.json")["rows"]:
        q, sc, zp = orc.quantize_rows_s8(np.array(row["x"], np.float32))
        assert sc[0] == np.float32(row["scale"]) and zp[0] == row["zp"]
        assert q[0].tolist() == row["q"]


def _adversarial_rows(rng, K):
    rows = [rng.standard_normal(K).astype(np.float32),
            (rng.standard_normal(K) * 1e-3 + 5).astype(np.float32),      # all positive
            (-rng.random(K) * 40).astype(np.float32),                      # all negative
            rng.uniform(-1e4, 3e-3, K).astype(np.float32),
            np.zeros(K, np.float32)]
    r = rng.standard_normal(K).astype(np.float32)
    r[::3] = 0.0
    rows.append(r)
    return np.stack(rows)


def test_o5_properties(orc):
    rng = np.random.default_rng(15)
    X = _adversarial_rows(rng, 257)
    Q, S, Z = orc.quantize_rows_s8(X)
    for x, q, s, z in zip(X, Q, S, Z):
        q = q.astype(np.int64)
        assert -128 <= z <= 127
        assert np.all(q[x == 0] == z)                               # real zero is exact
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order]) >= 0)                       # monotone
        deq = (q - z).astype(np.float64) * np.float64(s)
        assert np.all(np.abs(deq - x) <= np.float64(s) * (1 + 1e-6))  # within one step
        if np.any(x != 0):
            assert q[np.argmin(x)] in (-128, -127) or x.min() >= 0
            assert s == np.float32((np.float32(max(0, x.max())) - np.float32(min(0, x.min()))) / np.float32(255))


def test_o5_exact_ties_round_to_even(orc):
    # scale 1 (range 255), zp -128: x = j + 1/2 is an exact tie.
    x = np.array([0.0, 255.0] + [j + 0.5 for j in range(0, 254, 3)], np.float32)
    q, s, z = orc.quantize_rows_s8(x)
    assert s[0] == 1.0 and z[0] == -128
    for xv, qv in zip(x[2:], q[0, 2:]):
        j = int(xv - 0.5)
        assert qv == (j if j % 2 == 0 else j + 1) - 128


def test_o5_brute_force_grid(orc):
    """Every row over a small grid of values: codes equal exact rational
    rounding of x/scale (scale taken as the oracle's f32 value) whenever the
    quotient is not within f32 rounding of a tie."""
    vals = np.array([-3.0, -1.25, -0.5, 0.0, 0.75, 1.0, 2.5, 7.0], np.float32)
    import itertools
    for row in itertools.product(vals, repeat=3):
        x = np.array(row, np.float32)
        q, s, z = orc.quantize_rows_s8(x)
        sf = Fraction(float(s[0]))
        for xv, qv in zip(x, q[0]):
            ex = Fraction(float(xv)) / sf
            frac = ex - math.floor(ex)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 16):
                continue
            want = max(-128, min(127, round(ex) + int(z[0])))
            assert qv == want


# ------------------------------------------------------------------ O5s
def test_o5s_special_rows(orc):
    """All-zero row: scale 1, codes 0.  The largest magnitude maps to +-127."""
    q, s = orc.quantize_rows_s8_sym(np.zeros((1, 7), np.float32))
    assert s[0] == 1.0 and not q.any()
    rng = np.random.default_rng(41)
    x = rng.normal(0, 3, (5, 33)).astype(np.float32)
    q, s = orc.quantize_rows_s8_sym(x)
    for r in range(5):
        i = int(np.argmax(np.abs(x[r])))
        assert q[r, i] == (127 if x[r, i] > 0 else -127)
        assert s[r] == np.float32(np.abs(x[r]).max()) / np.float32(127)
    assert q.min() >= -127 and q.max() <= 127


def test_o5s_odd_symmetry_monotone_and_error_bound(orc):
    rng = np.random.default_rng(42)
    x = rng.uniform(-5, 5, (3, 101)).astype(np.float32)
    q, s = orc.quantize_rows_s8_sym(x)
    qn, sn = orc.quantize_rows_s8_sym(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for r in range(3):
        order = np.argsort(x[r], kind="stable")
        assert (np.diff(q[r][order].astype(int)) >= 0).all()
        err = np.abs(q[r].astype(np.float64) * float(s[r]) - x[r].astype(np.float64))
        assert (err <= 0.5 * float(s[r]) * (1 + 1e-5)).all()


def test_o5s_exact_ties_round_to_even(orc):
    """amax = 127/128 gives scale = 2^-7 exactly, so x = (j + 1/2) * 2^-7 is an
    exact tie of x/scale: it must round to the even neighbour."""
    j = np.array([0, 1, 2, 3, 4, 125, -1, -2, -3, -126], np.float64)
    x = np.concatenate([[127.0 / 128.0], (j + 0.5) / 128.0]).astype(np.float32)
    q, s = orc.quantize_rows_s8_sym(x)
    assert s[0] == np.float32(2.0 ** -7)
    # ties: 0.5->0, 1.5->2, 2.5->2, 3.5->4, 4.5->4, 125.5->126, -0.5->0, -1.5->-2,
    # -2.5->-2, -125.5->-126
    want = [127] + [0, 2, 2, 4, 4, 126, 0, -2, -2, -126]
    assert q[0].tolist() == want


def test_o5s_brute_force_grid(orc):
    """Rows over a value grid: codes equal the exact rational rounding of
    x/scale (with the oracle's f32 scale) away from f32-rounding distance of
    a tie, and the scale is the f32 quotient max|x| / 127."""
    vals = np.array([-3.0, -1.25, -0.5, 0.0, 0.75, 1.0, 2.5, 7.0], np.float32)
    import itertools
    for row in itertools.product(vals, repeat=3):
        x = np.array(row, np.float32)
        q, s = orc.quantize_rows_s8_sym(x)
        amax = np.float32(np.abs(x).max())
        assert s[0] == (np.float32(amax / np.float32(127)) if amax > 0 else 1.0)
        sf = Fraction(float(s[0]))
        for xv, qv in zip(x, q[0]):
            ex = Fraction(float(xv)) / sf
            frac = ex - math.floor(ex)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 16):
                continue
            assert qv == max(-127, min(127, round(ex)))


# ------------------------------------------------------------------ O6
def test_o6_single_group_closed_form(orc):
    rng = np.random.default_rng(16)
    qa = _rand_i8(rng, (3, 32))
    qw = _rand_i8(rng, (5, 32), -8, 7)
    sa = np.array([0.5, 0.25, 0.125], np.float32)
    za = np.array([3, -7, 0], np.int32)
    sw = np.array([[2.0 ** -6], [2.0 ** -7], [2.0 ** -5], [2.0 ** -8], [2.0 ** -6]], np.float32)
    bias = np.array([0.5, -0.25, 0, 1, -1], np.float32)
    Y = orc.a8w4_blockwise(qa, sa, za, qw, sw, bias, -1e9, 1e9)
    D = (qa.astype(np.int64) - za[:, None]) @ qw.T.astype(np.int64)
    want = sa[:, None].astype(np.float64) * sw[:, 0][None, :] * D + bias[None, :]
    assert np.array_equal(Y, want.astype(np.float32))   # powers of two: exact


def test_o6_uniform_scales_reduce_to_integer_gemm(orc):
    rng = np.random.default_rng(17)
    qa = _rand_i8(rng, (4, 96))
    qw = _rand_i8(rng, (6, 96), -8, 7)
    sw = np.full((6, 3), 2.0 ** -4, np.float32)
    Y = orc.a8w4_blockwise(qa, np.ones(4, np.float32), np.zeros(4, np.int32), qw, sw, None, -1e9, 1e9)
    want = (qa.astype(np.int64) @ qw.T.astype(np.int64)) * 2.0 ** -4
    assert np.array_equal(Y, want.astype(np.float32))


def test_o6_each_group_uses_its_own_scale(orc):
    K, G = 128, 4
    qa = np.ones((1, K), np.int8)
    sw = np.array([[1.0, 10.0, 100.0, 1000.0]], np.float32)
    for g in range(G):
        qw = np.zeros((1, K), np.int8)
        qw[0, g * 32 + 5] = 3
        Y = orc.a8w4_blockwise(qa, np.ones(1, np.float32), np.zeros(1, np.int32), qw, sw, None, -1e9, 1e9)
        assert Y[0, 0] == 3 * sw[0, g]


def test_o6_zero_point_and_clamp(orc):
    qa = np.full((1, 64), -9, np.int8)
    qw = np.full((2, 64), 7, np.int8)
    sw = np.full((2, 2), 0.01, np.float32)
    bias = np.array([0.25, 9.0], np.float32)
    Y = orc.a8w4_blockwise(qa, np.array([0.3], np.float32), np.array([-9], np.int32), qw, sw, bias, -6, 6)
    assert Y.tolist() == [[0.25, 6.0]]            # qa == za contributes real zero
    Y = orc.a8w4_blockwise(qa, np.array([1.0], np.float32), np.array([0], np.int32), qw, sw, -bias, -6, 6)
    assert Y[0, 1] == -6.0


def test_o6_brute_force_against_exact_rationals(orc):
    rng = np.random.default_rng(18)
    for _ in range(20):
        M, N, G = rng.integers(1, 4), rng.integers(1, 5), rng.integers(1, 4)
        K = int(G * 32 - rng.integers(0, 31))
        qa = _rand_i8(rng, (M, K))
        qw = _rand_i8(rng, (N, K), -8, 7)
        sa = rng.uniform(0.001, 0.1, M).astype(np.float32)
        za = rng.integers(-128, 128, M).astype(np.int32)
        sw = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
        bias = rng.uniform(-1, 1, N).astype(np.float32)
        Y = orc.a8w4_blockwise(qa, sa, za, qw, sw, bias, -6, 6)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for g in range(G):
                    d = sum((int(qa[m, k]) - int(za[m])) * int(qw[n, k]) for k in range(g * 32, min(K, g * 32 + 32)))
                    tot += Fraction(float(sw[n, g])) * d
                y = Fraction(float(sa[m])) * tot + Fraction(float(bias[n]))
                y = min(max(y, Fraction(-6)), Fraction(6))
                ulp = np.spacing(np.float32(abs(float(y)))) if y != 0 else np.float32(1e-45)
                assert abs(Fraction(float(Y[m, n])) - y) <= Fraction(float(ulp))


def test_o6_full_path_from_float_activations(orc):
    d = synth.a8w4(synth.BASE_SEED + 99, 2, 16, 64)
    Y = orc.a8w4_forward(d["X"], d["W"], d["sw"], d["bias"], -6, 6)
    # dequantized-activation float reference: the quantization error bound
    qa, sa, za = orc.quantize_rows_s8(d["X"])
    Xd = (qa.astype(np.float64) - za[:, None]) * sa[:, None]
    Wd = d["W"].astype(np.float64) * np.repeat(d["sw"].astype(np.float64), 32, axis=1)
    want = np.clip(Xd @ Wd.T + d["bias"], -6, 6)
    assert np.allclose(Y, want, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ O7
def _hdr(blob):
    h = blob[:256]
    u32 = h[:16].view(np.uint32)
    i64 = h[16:104].view(np.int64)
    keys = ["N", "K", "Npad", "Kpad", "group", "data_off", "data_bytes", "scale_off",
            "sum_off", "zp_off", "total_bytes"]
    d = dict(zip(keys, (int(v) for v in i64)))
    d.update(magic=int(u32[0]), version=int(u32[1]), format=int(u32[2]), scheme=int(u32[3]),
             has_zp=int(h[104:108].view(np.int32)[0]))
    d["scale_min"], d["scale_max"] = (float(v) for v in h[112:120].view(np.float32))
    assert not h[108:112].any() and not h[120:].any()
    if d["format"] != 1:
        assert d["scale_min"] == d["scale_max"] == 0.0
    return d


@pytest.mark.parametrize("N,K", [(1, 1), (70, 129), (64, 64), (65, 200), (3, 576)])
def test_o7_s8_blob_decodes_back(orc, N, K):
    rng = np.random.default_rng(19)
    W = _rand_i8(rng, (N, K))
    sc = rng.uniform(0.001, 0.01, N).astype(np.float32)
    zp = rng.integers(-3, 3, N).astype(np.int32)
    blob = orc.pack_s8_ref(W, sc, zp, per_channel=True)
    h = _hdr(blob)
    assert h["magic"] == 0x4B505149 and h["format"] == 1 and h["scheme"] == 1
    assert (h["N"], h["K"]) == (N, K)
    assert h["Npad"] % 64 == 0 and h["Kpad"] % 64 == 0 and h["Npad"] >= N and h["Kpad"] >= K
    assert h["total_bytes"] == blob.size == orc.lib().orc_packed_s8_bytes(N, K)
    # 32x32 sub-tiles: (n block, k block, row in block, byte in block) -> [n, k]
    data = blob[h["data_off"]:h["data_off"] + h["data_bytes"]].view(np.int8)
    data = data.reshape(h["Npad"] // 32, h["Kpad"] // 32, 32, 32).transpose(0, 2, 1, 3)
    data = data.reshape(h["Npad"], h["Kpad"])
    assert np.array_equal(data[:N, :K], W)
    assert not data[N:].any() and not data[:, K:].any()
    scales = blob[h["scale_off"]:h["scale_off"] + 4 * h["Npad"]].view(np.float32)
    assert np.array_equal(scales[:N], sc) and not scales[N:].any()
    cs = blob[h["sum_off"]:h["sum_off"] + 4 * h["Npad"]].view(np.int32)
    assert np.array_equal(cs[:N], W.astype(np.int64).sum(1)) and not cs[N:].any()
    zz = blob[h["zp_off"]:h["zp_off"] + 4 * h["Npad"]].view(np.int32)
    assert np.array_equal(zz[:N], zp) and h["has_zp"] == int(zp.any())
    assert (h["scale_min"], h["scale_max"]) == (float(sc.min()), float(sc.max()))
    # same blob from a [K, N] source view
    assert np.array_equal(orc.pack_s8_ref(np.ascontiguousarray(W.T).T, sc, zp), blob)


@pytest.mark.parametrize("N,K", [(1, 32), (5, 100), (64, 4096 // 8), (130, 64), (3, 300)])
def test_o7_s4_blob_decodes_back(orc, N, K):
    rng = np.random.default_rng(20)
    W = _rand_i8(rng, (N, K), -8, 7)
    G = (K + 31) // 32
    sw = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    blob = orc.pack_s4_ref(W, sw, 32)
    h = _hdr(blob)
    Kp = (K + 127) // 128 * 128
    Gp = Kp // 32
    assert h["format"] == 2 and h["group"] == 32 and h["Kpad"] == Kp
    # decode with numpy axes: (tile of 16 rows, block of 128 K, row in tile, c, t, j)
    #   -> row 16*tile + r, k = 128*block + 32t + 8c + [j | 4+j]
    raw = blob[h["data_off"]:h["data_off"] + h["data_bytes"]].reshape(
        h["Npad"] // 16, Kp // 128, 16, 4, 4, 4).transpose(0, 2, 1, 3, 4, 5)
    raw = raw.reshape(h["Npad"], Kp // 128, 4, 4, 4)
    lo = (raw & 0xF).astype(np.int16)
    hi = (raw >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    dec = np.concatenate([lo, hi], axis=4)              # (row, block, c, t, 8)
    dec = dec.transpose(0, 1, 3, 2, 4).reshape(h["Npad"], Kp)   # -> (row, block, t, c, 8)
    assert np.array_equal(dec[:N, :K], W) and not dec[N:].any() and not dec[:, K:].any()
    # scales: (tile of 16 rows, quad of 4 groups, row in tile, group in quad)
    sc = blob[h["scale_off"]:h["scale_off"] + 4 * h["Npad"] * Gp].view(np.float32)
    sc = sc.reshape(h["Npad"] // 16, Gp // 4, 16, 4).transpose(0, 2, 1, 3).reshape(h["Npad"], Gp)
    assert np.array_equal(sc[:N, :G], sw) and not sc[N:].any() and not sc[:, G:].any()
    Wp = np.zeros((N, G * 32), np.int64)
    Wp[:, :K] = W
    gs = Wp.reshape(N, G, 32).sum(2)
    ws = blob[h["sum_off"]:h["sum_off"] + 4 * h["Npad"]].view(np.float32)
    want = np.array([math.fsum(float(a) * float(b) for a, b in zip(sw[n], gs[n])) for n in range(N)],
                    np.float64).astype(np.float32)
    assert np.array_equal(ws[:N], want) and not ws[N:].any()


# ------------------------------------------------------------------ O9
def test_o9_dequant_is_the_correctly_rounded_product(orc):
    """Each value is s*(q - z) rounded once to f32: the fp64 product of a
    24-bit scale and a 9-bit integer is exact, so casting it to f32 is the
    correctly rounded result."""
    rng = np.random.default_rng(91)
    W = _rand_i8(rng, (7, 45))
    s = rng.uniform(1e-4, 1e-1, 7).astype(np.float32)
    z = rng.integers(-128, 128, 7).astype(np.int32)
    got = orc.dequant_weights_s8(W, s, z)
    want = (s.astype(np.float64)[:, None] * (W.astype(np.int64) - z[:, None])).astype(np.float32)
    assert got.dtype == np.float32 and np.array_equal(got, want)
    # scale per channel, not per k: a transposed scale vector changes row 0
    assert not np.array_equal(got[0], orc.dequant_weights_s8(W, s[::-1], z)[0])
    W4 = _rand_i8(rng, (5, 100), -8, 7)
    sw = rng.uniform(1e-3, 1e-2, (5, 4)).astype(np.float32)
    got4 = orc.dequant_weights_s4(W4, sw, 32)
    for n in range(5):
        for k in range(100):
            assert got4[n, k] == np.float32(float(sw[n, k // 32]) * int(W4[n, k]))


# ------------------------------------------------------------------ O6b
def test_o6b_bf16_rounding_matches_torch_cast(orc):
    """Round to nearest bf16, ties to even: the same values as torch's
    float32 -> bfloat16 conversion (a library routine), over random scales
    and hand-made ties."""
    import torch
    rng = np.random.default_rng(61)
    x = np.concatenate([rng.uniform(1e-4, 1.0, 5000), rng.uniform(0.002, 0.02, 5000),
                        np.exp(rng.uniform(-30, 30, 2000))]).astype(np.float32)
    got = orc.round_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 0.75 + 2 ** -9, 3 + 2 ** -7], np.float32)
    assert orc.round_bf16(ties).tolist() == [1.0, 1 + 2 ** -6, 0.75, 3.0]


def test_o6b_bf16_rounding_properties(orc):
    rng = np.random.default_rng(62)
    x = np.sort(rng.uniform(1e-3, 10.0, 20000).astype(np.float32))
    y = orc.round_bf16(x)
    assert np.all(np.diff(y) >= 0)                                  # monotone
    assert np.array_equal(orc.round_bf16(y), y)                     # idempotent
    assert np.all(np.abs(y.astype(np.float64) / x - 1) <= 2.0 ** -8)  # half an ulp of 8 bits
    # the low 16 bits of a bf16 value are zero
    assert not np.any(y.view(np.uint32) & 0xFFFF)


# ------------------------------------------------------------------ O6c
def _o6c_inputs(rng, M, N, K, G):
    qa = _rand_i8(rng, (M, K))
    sa = rng.uniform(0.01, 0.1, M).astype(np.float32)
    za = rng.integers(-128, 128, M).astype(np.int32)
    qw = _rand_i8(rng, (N, K), -8, 7)
    sw = rng.uniform(0.002, 0.02, (N, G)).astype(np.float32)
    bw = rng.uniform(-0.05, 0.05, (N, G)).astype(np.float32)
    return qa, sa, za, qw, sw, bw


def test_o6c_zero_offsets_reduce_to_o6(orc):
    rng = np.random.default_rng(71)
    qa, sa, za, qw, sw, _ = _o6c_inputs(rng, 3, 9, 100, 4)
    bias = rng.uniform(-1, 1, 9).astype(np.float32)
    got = orc.a8w4_blockwise_asym(qa, sa, za, qw, sw, np.zeros_like(sw), bias, -6, 6)
    assert np.array_equal(got, orc.a8w4_blockwise(qa, sa, za, qw, sw, bias, -6, 6))


def test_o6c_closed_form_constant_operands(orc):
    # qa == 5, za == -3, q == -2, sw = 2^-6, bw = 2^-3, K = 96 (three groups):
    # every output is sa * K * (5+3) * (-2*2^-6 + 2^-3) + bias, exactly
    M, N, K = 2, 3, 96
    qa = np.full((M, K), 5, np.int8)
    qw = np.full((N, K), -2, np.int8)
    sw = np.full((N, 3), 2.0 ** -6, np.float32)
    bw = np.full((N, 3), 2.0 ** -3, np.float32)
    sa = np.array([0.5, 0.25], np.float32)
    za = np.array([-3, -3], np.int32)
    bias = np.array([1.0, -2.0, 0.0], np.float32)
    y = orc.a8w4_blockwise_asym(qa, sa, za, qw, sw, bw, bias, -1e9, 1e9)
    for m in range(M):
        for n in range(N):
            assert y[m, n] == np.float32(float(sa[m]) * K * 8 * (-2 * 2.0 ** -6 + 2.0 ** -3)
                                         + float(bias[n]))


def test_o6c_integer_zero_points_match_direct_sum(orc):
    """bw = -sw*zw with an integer zero point per group is the affine form
    sw*(q - zw): compare with the sum written out in exact rationals."""
    rng = np.random.default_rng(72)
    M, N, K, G = 2, 4, 70, 3
    qa, sa, za, qw, sw, _ = _o6c_inputs(rng, M, N, K, G)
    sw = (2.0 ** -rng.integers(4, 9, (N, G))).astype(np.float32)   # powers of two: exact
    zw = rng.integers(-8, 8, (N, G))
    bw = (-sw * zw).astype(np.float32)
    y = orc.a8w4_blockwise_asym(qa, sa, za, qw, sw, bw, None, -1e30, 1e30)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                g = k // 32
                s += (int(qa[m, k]) - int(za[m])) * Fraction(float(sw[n, g])) \
                    * (int(qw[n, k]) - int(zw[n, g]))
            exact = Fraction(float(sa[m])) * s
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 23) \
                + Fraction(1, 2 ** 60)


def test_o6c_brute_force_rational(orc):
    rng = np.random.default_rng(73)
    M, N, K, G = 3, 5, 45, 2
    qa, sa, za, qw, sw, bw = _o6c_inputs(rng, M, N, K, G)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    y = orc.a8w4_blockwise_asym(qa, sa, za, qw, sw, bw, bias, -1e30, 1e30)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                g = k // 32
                w = Fraction(float(sw[n, g])) * int(qw[n, k]) + Fraction(float(bw[n, g]))
                s += (int(qa[m, k]) - int(za[m])) * w
            exact = Fraction(float(sa[m])) * s + Fraction(float(bias[n]))
            err = abs(Fraction(float(y[m, n])) - exact)
            assert err <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 40)
    # the offsets are per (channel, group): moving one group's offset changes
    # only that channel
    bw2 = bw.copy()
    bw2[1, 1] += 0.01
    y2 = orc.a8w4_blockwise_asym(qa, sa, za, qw, sw, bw2, bias, -1e30, 1e30)
    assert np.array_equal(np.delete(y2, 1, axis=1), np.delete(y, 1, axis=1))
    assert not np.array_equal(y2[:, 1], y[:, 1])


def test_o9_asymmetric_dequant_adds_the_group_offset(orc):
    rng = np.random.default_rng(93)
    W4 = _rand_i8(rng, (3, 70), -8, 7)
    sw = rng.uniform(1e-3, 1e-2, (3, 3)).astype(np.float32)
    bw = rng.uniform(-0.05, 0.05, (3, 3)).astype(np.float32)
    got = orc.dequant_weights_s4(W4, sw, 32, bw)
    for n in range(3):
        for k in range(70):
            p = np.float32(float(sw[n, k // 32]) * int(W4[n, k]))     # exact product, one rounding
            assert got[n, k] == np.float32(float(p) + float(bw[n, k // 32]))


# ------------------------------------------------------------------ O5b / O6d
def test_o5b_blocks_are_independent_rows(orc):
    """Each block of a row is quantized exactly as O5 quantizes that block
    given as a row of its own; block = K is O5 itself."""
    rng = np.random.default_rng(51)
    X = (rng.standard_normal((3, 100)) * rng.uniform(0.1, 10, (3, 1))).astype(np.float32)
    X[1, 32:64] = 0.0                       # an all-zero block: scale 1, zp 0
    X[2, 64:96] = np.abs(X[2, 64:96]) + 1   # an all-positive block
    q, sc, zp = orc.quantize_rows_s8_blocked(X, 32)
    assert sc.shape == (3, 4) and zp.shape == (3, 4)
    for m in range(3):
        for g in range(4):
            qq, ss, zz = orc.quantize_rows_s8(X[m, 32 * g:32 * g + 32])
            assert np.array_equal(q[m, 32 * g:32 * g + 32], qq[0])
            assert sc[m, g] == ss[0] and zp[m, g] == zz[0]
    assert sc[1, 1] == 1.0 and zp[1, 1] == 0 and not q[1, 32:64].any()
    qa, sa, za = orc.quantize_rows_s8(X)
    qb, sb, zb = orc.quantize_rows_s8_blocked(X, 100)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb[:, 0]) and np.array_equal(za, zb[:, 0])
    # finer blocks never quantize worse: every block's error bound is its own scale
    err = np.abs((q.astype(np.float64) - np.repeat(zp, 32, 1)[:, :100]) *
                 np.repeat(sc, 32, 1)[:, :100] - X)
    assert np.all(err <= np.repeat(sc, 32, 1)[:, :100])


def test_o6d_uniform_activation_params_reduce_to_o6(orc):
    rng = np.random.default_rng(52)
    M, N, K = 3, 7, 96
    qa = _rand_i8(rng, (M, K))
    qw = _rand_i8(rng, (N, K), -8, 7)
    sw = rng.uniform(0.002, 0.02, (N, 3)).astype(np.float32)
    sa = rng.uniform(0.01, 0.05, M).astype(np.float32)
    za = rng.integers(-100, 100, M).astype(np.int32)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    got = orc.a8w4_blockwise_blockq(qa, np.repeat(sa[:, None], 3, 1), np.repeat(za[:, None], 3, 1),
                                    qw, sw, bias, -6, 6)
    want = orc.a8w4_blockwise(qa, sa, za, qw, sw, bias, -6, 6)
    assert np.max(np.abs(got.astype(np.float64) - want)) <= 1e-6 * np.max(np.abs(want))


def test_o6d_brute_force_rational(orc):
    rng = np.random.default_rng(53)
    M, N, K = 2, 4, 70
    qa = _rand_i8(rng, (M, K))
    qw = _rand_i8(rng, (N, K), -8, 7)
    sw = rng.uniform(0.002, 0.02, (N, 3)).astype(np.float32)
    sa = rng.uniform(0.01, 0.05, (M, 3)).astype(np.float32)
    za = rng.integers(-128, 128, (M, 3)).astype(np.int32)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    y = orc.a8w4_blockwise_blockq(qa, sa, za, qw, sw, bias, -1e30, 1e30)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                g = k // 32
                s += Fraction(float(sa[m, g])) * Fraction(float(sw[n, g])) \
                    * (int(qa[m, k]) - int(za[m, g])) * int(qw[n, k])
            exact = s + Fraction(float(bias[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 23) \
                + Fraction(1, 2 ** 40)
    # a block's activation zero point touches only its own group
    za2 = za.copy()
    za2[0, 2] += 5
    y2 = orc.a8w4_blockwise_blockq(qa, sa, za2, qw, sw, bias, -1e30, 1e30)
    assert np.array_equal(y2[1], y[1]) and not np.array_equal(y2[0], y[0])


# ------------------------------------------------------------------ O6 on int8 blocks
@pytest.mark.parametrize("group", [64, 128])
def test_o6_int8_weight_blocks_against_exact_rationals(orc, group):
    """O6's definition read for block-quantized int8 weights: full int8
    values, one scale per block of 64 or 128 K."""
    rng = np.random.default_rng(group)
    M, N, K = 2, 3, 2 * group + 37
    G = (K + group - 1) // group
    qa = _rand_i8(rng, (M, K))
    qw = _rand_i8(rng, (N, K))                       # full [-128, 127]
    sa = rng.uniform(0.001, 0.1, M).astype(np.float32)
    za = rng.integers(-128, 128, M).astype(np.int32)
    sw = rng.uniform(1e-4, 1e-3, (N, G)).astype(np.float32)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    Y = orc.a8w4_blockwise(qa, sa, za, qw, sw, bias, -1e30, 1e30, group)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(G):
                d = sum((int(qa[m, k]) - int(za[m])) * int(qw[n, k])
                        for k in range(g * group, min(K, g * group + group)))
                tot += Fraction(float(sw[n, g])) * d
            y = Fraction(float(sa[m])) * tot + Fraction(float(bias[n]))
            assert abs(Fraction(float(Y[m, n])) - y) <= abs(y) * Fraction(1, 2 ** 23) \
                + Fraction(1, 2 ** 40)


# ------------------------------------------------------------------ O4c
def test_o4c_single_block_is_o4_scaled(orc):
    """One block spanning every input channel: sx * sw[oc] * O4's integer
    accumulator + bias (power-of-two scales keep it exact)."""
    rng = np.random.default_rng(41)
    X = _rand_i8(rng, (2, 7, 6, 8))
    Wt = _rand_i8(rng, (5, 8, 3, 3), -127, 127)
    sw = (2.0 ** -rng.integers(6, 10, (5, 1))).astype(np.float32)
    bias = np.array([0.5, -1.0, 0.0, 2.0, -0.25], np.float32)
    y = orc.conv2d_blockwise_f32(X, 7, 0.125, Wt, 8, sw, (1, 1), (1, 1, 1, 1), bias)
    acc = orc.conv2d_direct(X, 7, Wt, (1, 1), (1, 1, 1, 1))
    want = 0.125 * sw[:, 0].astype(np.float64) * acc + bias
    assert np.array_equal(y, want.astype(np.float32))


def test_o4c_blocks_are_input_channel_ranges(orc):
    """Scaling one block's scale by 2 equals adding that block's own
    contribution once more; the blocks split the input channels, each over
    every kernel tap (a weight zeroed outside block 1 isolates it)."""
    rng = np.random.default_rng(42)
    X = _rand_i8(rng, (1, 6, 6, 12))
    Wt = _rand_i8(rng, (3, 12, 3, 3), -127, 127)
    sw = (2.0 ** -rng.integers(6, 9, (3, 3))).astype(np.float32)    # icb = 4: 3 blocks
    base = orc.conv2d_blockwise_f32(X, -5, 0.5, Wt, 4, sw, (1, 1), (1, 1, 1, 1)).astype(np.float64)
    only1 = Wt.copy()
    only1[:, :4] = 0
    only1[:, 8:] = 0
    part1 = orc.conv2d_blockwise_f32(X, -5, 0.5, only1, 4, sw, (1, 1), (1, 1, 1, 1))
    sw2 = sw.copy()
    sw2[:, 1] *= 2
    twice = orc.conv2d_blockwise_f32(X, -5, 0.5, Wt, 4, sw2, (1, 1), (1, 1, 1, 1))
    assert np.array_equal(twice, (base + part1).astype(np.float32))
    with pytest.raises(Exception):
        orc.conv2d_blockwise_f32(X, -5, 0.5, Wt, 5, np.ones((3, 2), np.float32))   # 12 % 5


def test_o4c_brute_force_rational(orc):
    rng = np.random.default_rng(43)
    X = _rand_i8(rng, (1, 4, 5, 4))
    Wt = _rand_i8(rng, (2, 4, 2, 3), -127, 127)
    sw = rng.uniform(1e-3, 1e-2, (2, 2)).astype(np.float32)
    bias = rng.uniform(-1, 1, 2).astype(np.float32)
    zx, sx = 9, np.float32(0.03)
    y = orc.conv2d_blockwise_f32(X, zx, sx, Wt, 2, sw, (1, 2), (1, 0, 0, 2), bias, (2, 1))
    OH, OW = orc.conv_out_dims(4, 5, 2, 3, (1, 2), (1, 0, 0, 2), (2, 1))
    for oy in range(OH):
        for ox in range(OW):
            for oc in range(2):
                s = Fraction(0)
                for ky in range(2):
                    for kx in range(3):
                        iy, ix = oy * 1 + ky * 2 - 1, ox * 2 + kx * 1 - 0
                        for ic in range(4):
                            xv = int(X[0, iy, ix, ic]) if 0 <= iy < 4 and 0 <= ix < 5 else zx
                            s += Fraction(float(sw[oc, ic // 2])) * (xv - zx) * int(Wt[oc, ic, ky, kx])
                exact = Fraction(float(sx)) * s + Fraction(float(bias[oc]))
                assert abs(Fraction(float(y[0, oy, ox, oc])) - exact) <= \
                    abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 40)
