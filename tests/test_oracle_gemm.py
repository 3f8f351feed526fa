"""Pins of the oracle's integer GEMM (O1), tiled model (O2) and requantization
(O3) to facts fixed outside the oracle: the worked example's printed tile
numbers, the INT32 bound, textbook identities, exact rational rounding and
brute force.  CPU only."""
import itertools
import json
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


# ------------------------------------------------------------------ O1
def test_o1_matches_library_matmul_without_zero_points(orc):
    rng = np.random.default_rng(1)
    A, B = _rand_i8(rng, (13, 37)), _rand_i8(rng, (37, 11))
    acc = orc.gemm_affine(A, 0, B, 0)
    assert np.array_equal(acc, A.astype(np.int64) @ B.astype(np.int64))


def test_o1_expanded_identity_brute_force(orc):
    """sum (a-zA)(b-zB) == sum ab - zB sum a - zA sum b + K zA zB, over every
    tiny shape up to 4 and a sweep of zero points (catches a dropped term or a
    wrong sign anywhere in the zero-point handling)."""
    rng = np.random.default_rng(2)
    for M, N, K in itertools.product(range(1, 5), repeat=3):
        A, B = _rand_i8(rng, (M, K)), _rand_i8(rng, (K, N))
        zA = int(rng.integers(-128, 128))
        zB = rng.integers(-128, 128, size=N).astype(np.int32)
        bias = rng.integers(-1000, 1001, size=N).astype(np.int32)
        A64, B64 = A.astype(np.int64), B.astype(np.int64)
        want = (A64 @ B64 - np.outer(A64.sum(1), zB) - zA * B64.sum(0)[None, :]
                + K * zA * zB[None, :].astype(np.int64) + bias[None, :])
        assert np.array_equal(orc.gemm_affine(A, zA, B, zB, bias), want)


def test_o1_strided_and_transposed_operands(orc):
    rng = np.random.default_rng(3)
    A = _rand_i8(rng, (9, 40))[:, ::2]          # non-unit K stride
    Bnk = _rand_i8(rng, (7, 20))                 # [N, K] source
    acc_nk = orc.gemm_affine(A, 4, Bnk, -3, b_is_nk=True)
    acc_kn = orc.gemm_affine(np.ascontiguousarray(A), 4, np.ascontiguousarray(Bnk.T), -3)
    want = (A.astype(np.int64) - 4) @ (Bnk.T.astype(np.int64) + 3)
    assert np.array_equal(acc_nk, want) and np.array_equal(acc_kn, want)


def test_o1_int32_bound_is_attained(orc):
    g = _gold("int32_bound.json")
    K = g["K"]
    assert orc.int32_bound(K, 0) == g["bound_without_bias"]
    assert orc.int32_bound(K, 7) == g["bound_without_bias"] + 7
    c = g["attaining_case"]
    A = np.full((1, K), c["A"], np.int8)
    B = np.full((K, 1), c["B"], np.int8)
    acc = orc.gemm_affine(A, c["zA"], B, c["zB"])
    assert acc[0, 0] == c["acc"] == -g["bound_without_bias"]
    assert g["max_abs_operand"] ** 2 == g["max_abs_product"]


def test_o1_zero_point_padding_of_k_is_invariant(orc):
    """Padding K 129 -> 256 with A=zA and B=zB leaves every output unchanged."""
    d = synth.gemm_affine_per_tensor()
    A, B = d["A"], d["B"]
    acc = orc.gemm_affine(A, d["zA"], B, d["zB"], d["bias"])
    Ap = np.full((A.shape[0], 256), d["zA"], np.int8)
    Ap[:, :129] = A
    Bp = np.full((256, B.shape[1]), d["zB"], np.int8)
    Bp[:129] = B
    assert np.array_equal(orc.gemm_affine(Ap, d["zA"], Bp, d["zB"], d["bias"]), acc)
    # padding with integer 0 instead of the zero points is NOT neutral
    Az = np.zeros_like(Ap); Az[:, :129] = A
    Bz = np.zeros_like(Bp); Bz[:129] = B
    assert not np.array_equal(orc.gemm_affine(Az, d["zA"], Bz, d["zB"], d["bias"]), acc)


def test_o1_extra_rows_and_columns_do_not_touch_valid_outputs(orc):
    rng = np.random.default_rng(4)
    A, B = _rand_i8(rng, (10, 33)), _rand_i8(rng, (33, 6))
    acc = orc.gemm_affine(A, 1, B, 2)
    Ab = np.concatenate([A, _rand_i8(rng, (5, 33))])
    Bb = np.concatenate([B, _rand_i8(rng, (33, 3))], axis=1)
    assert np.array_equal(orc.gemm_affine(Ab, 1, Bb, 2)[:10, :6], acc)


def test_o1_points_agree_with_full(orc):
    rng = np.random.default_rng(5)
    A, Bnk = _rand_i8(rng, (20, 50)), _rand_i8(rng, (15, 50))
    zB = rng.integers(-5, 5, 15).astype(np.int32)
    bias = rng.integers(-9, 9, 15).astype(np.int32)
    full = orc.gemm_affine(A, -7, Bnk, zB, bias, b_is_nk=True)
    ms, ns = rng.integers(0, 20, 40), rng.integers(0, 15, 40)
    pts = orc.gemm_affine_points(ms, ns, A, -7, Bnk, zB, bias, b_is_nk=True)
    assert np.array_equal(pts, full[ms, ns])


# ------------------------------------------------------------------ O2
def test_o2_worked_example_numbers():
    import oracle
    g = _gold("npu_tiling_example.json")
    d = synth.gemm_affine_per_tensor()
    t = g["tile"]
    acc_t, st = oracle.gemm_tiled(d["A"], d["zA"], d["B"], d["zB"], d["bias"],
                                  t["Tm"], t["Tn"], t["Tk"])
    assert (st["tiles_m"], st["tiles_n"], st["tiles_k"]) == (g["tiles_m"], g["tiles_n"], g["tiles_k"])
    assert st["tiles"] == g["tiles"]
    assert st["effective_mac"] == g["effective_mac"]
    assert st["physical_slots"] == g["physical_slots"]
    assert round(100 * st["shape_efficiency"], 2) == g["shape_efficiency_percent_printed"]
    b = oracle.tile_budget(t["Tm"], t["Tn"], t["Tk"], 1, 4, t["reserve_bytes"])
    assert b["s_input"] == g["s_input_bytes"]
    assert b["s_acc"] == g["s_acc_bytes"]
    assert b["s_total"] == g["s_total_bytes"]
    # level 3 of the verification ladder: tiled model == full integer GEMM
    acc = oracle.gemm_affine(d["A"], d["zA"], d["B"], d["zB"], d["bias"])
    assert np.array_equal(acc_t, acc)


@pytest.mark.parametrize("tiles", [(1, 1, 1), (3, 5, 7), (16, 8, 4), (64, 64, 128)])
def test_o2_tiled_equals_full_for_any_tiling(orc, tiles):
    rng = np.random.default_rng(6)
    A, B = _rand_i8(rng, (23, 31)), _rand_i8(rng, (31, 17))
    zB = rng.integers(-128, 128, 17).astype(np.int32)
    bias = rng.integers(-1000, 1001, 17).astype(np.int32)
    full = orc.gemm_affine(A, 9, B, zB, bias)
    tiled, _ = orc.gemm_tiled(A, 9, B, zB, bias, *tiles)
    assert np.array_equal(tiled, full)


def test_o2_narrowing_every_k_block_changes_results(orc):
    """Requantizing each K block's partial sum to int8 and adding the int8
    results is not the contract: it must differ from requantizing once after
    all of K."""
    d = synth.gemm_affine_per_tensor()
    A, B = d["A"], d["B"]
    acc = orc.gemm_affine(A, d["zA"], B, d["zB"], d["bias"])
    once, _ = orc.requant_matrix(acc, d["sA"], d["sB"], d["s_out"], d["zp_out"], False)
    parts = [orc.gemm_affine(A[:, :128], d["zA"], B[:128], d["zB"], d["bias"]),
             orc.gemm_affine(A[:, 128:], d["zA"], B[128:], d["zB"])]
    narrowed = sum(orc.requant_matrix(p, d["sA"], d["sB"], d["s_out"], 0, False)[0].astype(np.int64)
                   for p in parts) + d["zp_out"]
    assert np.array_equal(parts[0] + parts[1], acc)
    assert not np.array_equal(np.clip(narrowed, -128, 127), once.astype(np.int64))


# ------------------------------------------------------------------ O3
def _rhe_fraction(x: Fraction) -> int:
    return round(x)  # Python rounds a Fraction half to even


def test_o3_power_of_two_multiplier_is_exact(orc):
    for s in [1, 2, 7, 15, 31, 40]:
        m0, sh = orc.requant_params(2.0 ** -s)
        assert m0 == 1 << 30 and sh == 30 + s
        for acc in [-(1 << 20) - 1, -12345, -3, -1, 0, 1, 2, 3, 99999, (1 << 24) + 1]:
            want = _rhe_fraction(Fraction(acc, 1 << s))
            assert orc.rshift_rhe(acc * m0, sh) == want


def test_o3_hand_worked_ties_round_to_even(orc):
    g = _gold("requant_ties.json")
    m0, sh = orc.requant_params(g["real_multiplier"])
    assert (m0, sh) == (g["m0"], g["shift"])
    for acc, q in g["cases"]:
        assert orc.requant_value(acc, m0, sh, 0, -1 << 20, 1 << 20) == q


def test_o3_multiplier_derivation_is_accurate(orc):
    """m0 / 2^shift approximates M to within 2^-31 relative (one Q31 rounding)."""
    rng = np.random.default_rng(7)
    for M in list(rng.uniform(1e-9, 0.999, 200)) + [1e-5, 4e-4, 0.5, 0.75, 1.0, 3.0, 1e3]:
        m0, sh = orc.requant_params(float(M))
        assert (1 << 30) <= m0 < (1 << 31)
        approx = Fraction(m0, 1 << sh)
        assert abs(approx - Fraction(float(M))) <= Fraction(float(M)) * Fraction(1, 1 << 31)


def test_o3_unsupported_multipliers(orc):
    import oracle
    for bad in [0.0, -1.0, float("inf"), float("nan"), 2.0 ** 31]:
        with pytest.raises(oracle.OracleError):
            orc.requant_params(bad)


def test_o3_contract_vs_ideal_exhaustive(orc):
    """Over every acc in [-2^16, 2^16] and several multipliers, the contract
    value equals the exactly rounded acc*M except at near-ties whose distance
    to the half point is below the multiplier's own error."""
    accs = range(-(1 << 16), (1 << 16) + 1, 1)
    for M in [4e-4, 1.0 / 3.0, 0.0123456, 2.5e-5, 0.999]:
        m0, sh = orc.requant_params(M)
        Mf = Fraction(M)
        err = abs(Fraction(m0, 1 << sh) - Mf)
        for acc in accs[:: 7 if M < 0.01 else 3]:
            got = orc.rshift_rhe(acc * m0, sh)
            exact = acc * Mf
            want = _rhe_fraction(exact)
            if got != want:
                frac = exact - (exact.numerator // exact.denominator)
                assert abs(frac - Fraction(1, 2)) <= abs(acc) * err, (M, acc)
            assert orc.ideal_rhe(acc, M) == want


def test_o3_saturation_relu_and_huge_shift(orc):
    m0, sh = orc.requant_params(0.5)
    assert orc.requant_value(10 ** 6, m0, sh, 0) == 127
    assert orc.requant_value(-(10 ** 6), m0, sh, 0) == -128
    assert orc.requant_value(-50, m0, sh, 5, lo=5) == 5           # ReLU: lower clamp at zp_out
    assert orc.requant_value(50, m0, sh, 5, lo=5) == 30
    m0, sh = orc.requant_params(2.0 ** -70)
    assert sh >= 63 and orc.requant_value(2 ** 31 - 1, m0, sh, -2) == -2
    acc = np.array([[10 ** 6, -(10 ** 6), 0, 3]], np.int64)
    out, _ = orc.requant_matrix(acc, 1.0, 0.5, 1.0, -3, True)
    assert out.tolist() == [[127, -3, -3, -1]]


def test_o3_matrix_is_per_column(orc):
    acc = np.array([[100, 100], [-7, 9]], np.int64)
    out, nd = orc.requant_matrix(acc, 1.0, np.array([0.5, 0.25], np.float32), 1.0, 0, False)
    assert out.tolist() == [[50, 25], [-4, 2]] and nd == 0


def test_fp64_matmul_formulation_equals_o1(orc):
    from oracle.matmul_f64 import gemm_affine_f64
    rng = np.random.default_rng(8)
    A, Bnk = _rand_i8(rng, (37, 300)), _rand_i8(rng, (29, 300))
    zB = rng.integers(-128, 128, 29).astype(np.int32)
    bias = rng.integers(-1000, 1001, 29).astype(np.int32)
    want = orc.gemm_affine(A, -11, Bnk, zB, bias, b_is_nk=True)
    assert np.array_equal(gemm_affine_f64(A, -11, Bnk, zB, bias), want)
    assert np.array_equal(gemm_affine_f64(A, -11, Bnk, zB, bias, rows=[3, 5]), want[[3, 5]])
    # the attained INT32 bound is reproduced exactly
    K = 129
    acc = gemm_affine_f64(np.full((1, K), -128, np.int8), 127, np.full((1, K), 127, np.int8), -128)
    assert acc[0, 0] == -K * 65025


# ------------------------------------------------------------------ O8
def _f32_ulp(x):
    x = np.float32(abs(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x)


def test_o8_closed_form_constant_operands(orc):
    # A == a, B == b everywhere: every accumulator is K*(a-zA)*(b-zB), and with
    # power-of-two scales and small integers the whole f32 result is exact.
    M, K, N = 3, 96, 5
    a, zA, zB = 7, -3, np.array([0, 1, -2, 5, 9], np.int32)
    A = np.full((M, K), a, np.int8)
    B = np.full((K, N), -4, np.int8)
    acc = orc.gemm_affine(A, zA, B, zB, None)
    sB = np.array([0.5, 0.25, 2.0, 1.0, 0.125], np.float32)
    bias = np.array([1.5, -2.0, 0.0, 3.25, -0.5], np.float32)
    y = orc.dequant_matrix_f32(acc, 0.25, sB, bias, -1e30, 1e30)
    for n in range(N):
        want = 0.25 * float(sB[n]) * K * (a - zA) * (-4 - int(zB[n])) + float(bias[n])
        assert (y[:, n] == np.float32(want)).all(), n


def test_o8_rounds_once_to_nearest_f32(orc):
    # Against the exact rational value: the fp64 intermediate keeps the result
    # within half an f32 ulp (plus a negligible fp64 term), never a full ulp.
    rng = np.random.default_rng(81)
    acc = rng.integers(-(2 ** 31) + 1, 2 ** 31 - 1, size=(4, 64)).astype(np.int64)
    sB = rng.uniform(1e-4, 1e-2, 64).astype(np.float32)
    bias = rng.uniform(-50, 50, 64).astype(np.float32)
    sA = np.float32(0.0123)
    y = orc.dequant_matrix_f32(acc, sA, sB, bias, -np.inf, np.inf)
    for m in range(4):
        for n in range(64):
            exact = (Fraction(float(sA)) * Fraction(float(sB[n])) * int(acc[m, n])
                     + Fraction(float(bias[n])))
            err = abs(Fraction(float(y[m, n])) - exact)
            assert err <= Fraction(_f32_ulp(float(exact))) * Fraction(1, 2) * (1 + Fraction(1, 1 << 20))


def test_o8_relu6_clamp_and_no_bias(orc):
    acc = np.array([[-100, 0, 3, 12, 13, 1000]], np.int64)
    y = orc.dequant_matrix_f32(acc, 0.5, 1.0, None, 0.0, 6.0)
    assert y.tolist() == [[0.0, 0.0, 1.5, 6.0, 6.0, 6.0]]
    # lo == hi forces every output to that value; lo > hi is rejected
    assert (orc.dequant_matrix_f32(acc, 0.5, 1.0, None, 2.0, 2.0) == 2.0).all()
    with pytest.raises(Exception):
        orc.dequant_matrix_f32(acc, 0.5, 1.0, None, 3.0, 2.0)


def test_o8_scale_and_bias_are_per_column(orc):
    acc = np.array([[10, 10, 10], [-4, 6, 8]], np.int64)
    y = orc.dequant_matrix_f32(acc, 1.0, np.array([1.0, 0.5, 0.25], np.float32),
                               np.array([0.0, 1.0, -1.0], np.float32), -1e9, 1e9)
    assert y.tolist() == [[10.0, 6.0, 1.5], [-4.0, 4.0, 1.0]]
