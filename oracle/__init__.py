"""Python view of the scalar C oracle (``oracle.c``).

Test infrastructure: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg import this package.  It is marshalling for the
C oracle (``oracle.c``) plus two small numpy definitions that are not in C:
O9, the dequantized weight values (one IEEE f32 product, plus the group
offset for asymmetric int4), and ``matmul_f64.py``, a second formulation of
O1 through an fp64 library matmul for full-size checks.  It never imports
the GPU library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` (next to the source)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class TileStats(C.Structure):
    _fields_ = [("tiles_m", C.c_int64), ("tiles_n", C.c_int64), ("tiles_k", C.c_int64),
                ("tiles", C.c_int64), ("effective_mac", C.c_int64),
                ("physical_slots", C.c_int64), ("shape_efficiency", C.c_double)]


class TileBudget(C.Structure):
    _fields_ = [("s_input", C.c_int64), ("s_acc", C.c_int64), ("s_reserve", C.c_int64),
                ("s_total", C.c_int64)]


_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_F = C.c_float
_D = C.c_double

_SIGS = {
    "orc_int32_bound": (_I64, [_I64, _I64]),
    "orc_gemm_affine": (C.c_int, [_I64, _I64, _I64, _P, _I64, _I64, _I32, _P, _I64, _I64, _P, _P, _P]),
    "orc_gemm_affine_points": (C.c_int, [_I64, _P, _P, _I64, _P, _I64, _I64, _I32, _P, _I64, _I64,
                                         _P, _P, _P]),
    "orc_tile_budget_of": (None, [_I64, _I64, _I64, _I64, _I64, _I64, C.POINTER(TileBudget)]),
    "orc_gemm_tiled": (C.c_int, [_I64, _I64, _I64, _P, _I64, _I64, _I32, _P, _I64, _I64, _P, _P,
                                 _I64, _I64, _I64, _P, C.POINTER(TileStats)]),
    "orc_real_multiplier": (_D, [_F, _F, _F]),
    "orc_requant_params": (C.c_int, [_D, C.POINTER(_I32), C.POINTER(_I32)]),
    "orc_rshift_rhe": (_I64, [_I64, _I32]),
    "orc_requant_value": (_I32, [_I64, _I32, _I32, _I32, _I32, _I32]),
    "orc_ideal_rhe": (_I64, [_I64, _D]),
    "orc_requant_matrix": (C.c_int, [_I64, _I64, _P, _F, _P, _F, _I32, _I32, _P, C.POINTER(_I64)]),
    "orc_conv2d_direct": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I32, _I64, _I64, _I64, _P, _I64,
                                    _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "orc_im2col": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I32, _I64, _I64, _I64, _I64, _I64, _I64,
                             _I64, _I64, _I64, _I64, _P]),
    "orc_quantize_row_s8": (None, [_P, _I64, _P, C.POINTER(_F), C.POINTER(_I32)]),
    "orc_quantize_rows_s8": (None, [_I64, _I64, _P, _I64, _P, _I64, _P, _P]),
    "orc_quantize_rows_s8_sym": (None, [_I64, _I64, _P, _I64, _P, _I64, _P]),
    "orc_round_bf16_array": (None, [_I64, _P, _P]),
    "orc_conv2d_blockwise_f32": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I32, _F, _I64, _I64, _I64,
                                           _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                           _I64, _P, _P, _F, _F, _P]),
    "orc_quantize_rows_s8_blocked": (None, [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I64]),
    "orc_a8w4_blockwise_blockq": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I64, _P, _P, _I64, _P,
                                            _I64, _P, _I64, _P, _F, _F, _P, _I64]),
    "orc_a8w4_blockwise_asym": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _I64, _P,
                                          _P, _I64, _P, _F, _F, _P, _I64]),
    "orc_dequant_matrix_f32": (C.c_int, [_I64, _I64, _P, _F, _P, _P, _F, _F, _P]),
    "orc_a8w4_blockwise": (C.c_int, [_I64, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _I64, _P, _I64,
                                     _P, _F, _F, _P, _I64]),
    "orc_packed_s8_bytes": (_I64, [_I64, _I64]),
    "orc_pack_s8_ref": (C.c_int, [_I64, _I64, _P, _I64, _I64, _I32, _P, _P, _P]),
    "orc_packed_s4_bytes": (_I64, [_I64, _I64, _I64]),
    "orc_pack_s4_ref": (C.c_int, [_I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _P]),
}


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = build(force=False)
            h = C.CDLL(path)
            for name, (res, args) in _SIGS.items():
                f = getattr(h, name)
                f.restype = res
                f.argtypes = args
            _lib = h
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _check(rc, what):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (what, rc))


def _elem_strides(a):
    return tuple(s // a.itemsize for s in a.strides)


def rows_in_threads(fn, X, *args, threads=None, chunk=None, **kw):
    """``fn(X[r0:r1], *args, **kw)`` over row ranges of ``X`` on host threads,
    concatenated along the first axis.  Every oracle function used this way
    treats rows independently, so the result is identical to one call; the
    C code runs without the interpreter lock, so the ranges run in
    parallel."""
    from concurrent.futures import ThreadPoolExecutor
    n = X.shape[0]
    threads = threads or min(16, os.cpu_count() or 1)
    chunk = chunk or max(1, -(-n // (4 * threads)))
    starts = range(0, n, chunk)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r0: fn(X[r0:r0 + chunk], *args, **kw), starts))
    return np.concatenate(parts, axis=0)


# ---------------------------------------------------------------- O1 / O2
def int32_bound(K, max_abs_bias):
    return lib().orc_int32_bound(int(K), int(max_abs_bias))


def gemm_affine(A, zA, B, zB, bias=None, b_is_nk=False):
    """acc[M,N] (int64) of sum_k (A[m,k]-zA)*(B[k,n]-zB[n]) + bias[n].

    ``A`` is [M,K]; ``B`` is [K,N], or [N,K] when ``b_is_nk``.  Any numpy
    strides are accepted (element strides are passed through)."""
    A = np.asarray(A, dtype=np.int8)
    B = np.asarray(B, dtype=np.int8)
    M, K = A.shape
    if b_is_nk:
        N = B.shape[0]
        b_sn, b_sk = _elem_strides(B)
    else:
        N = B.shape[1]
        b_sk, b_sn = _elem_strides(B)
    a_sm, a_sk = _elem_strides(A)
    zBv = _arr(np.broadcast_to(np.asarray(zB, dtype=np.int32), (N,)), np.int32)
    biasv = None if bias is None else _arr(bias, np.int32)
    out = np.zeros((M, N), dtype=np.int64)
    rc = lib().orc_gemm_affine(M, N, K, _ptr(A), a_sm, a_sk, int(zA), _ptr(B), b_sk, b_sn,
                               _ptr(zBv), _ptr(biasv), _ptr(out))
    _check(rc, "orc_gemm_affine")
    return out


def gemm_affine_points(ms, ns, A, zA, B, zB, bias=None, b_is_nk=False):
    A = np.asarray(A, dtype=np.int8)
    B = np.asarray(B, dtype=np.int8)
    K = A.shape[1]
    if b_is_nk:
        N = B.shape[0]
        b_sn, b_sk = _elem_strides(B)
    else:
        N = B.shape[1]
        b_sk, b_sn = _elem_strides(B)
    a_sm, a_sk = _elem_strides(A)
    ms = _arr(ms, np.int64)
    ns = _arr(ns, np.int64)
    zBv = _arr(np.broadcast_to(np.asarray(zB, dtype=np.int32), (N,)), np.int32)
    biasv = None if bias is None else _arr(bias, np.int32)
    out = np.zeros(ms.shape[0], dtype=np.int64)
    rc = lib().orc_gemm_affine_points(ms.shape[0], _ptr(ms), _ptr(ns), K, _ptr(A), a_sm, a_sk,
                                      int(zA), _ptr(B), b_sk, b_sn, _ptr(zBv), _ptr(biasv),
                                      _ptr(out))
    _check(rc, "orc_gemm_affine_points")
    return out


def tile_budget(Tm, Tn, Tk, in_elem_bytes=1, acc_elem_bytes=4, reserve=16384):
    b = TileBudget()
    lib().orc_tile_budget_of(Tm, Tn, Tk, in_elem_bytes, acc_elem_bytes, reserve, C.byref(b))
    return {"s_input": b.s_input, "s_acc": b.s_acc, "s_reserve": b.s_reserve, "s_total": b.s_total}


def gemm_tiled(A, zA, B, zB, bias, Tm, Tn, Tk):
    A = np.asarray(A, dtype=np.int8)
    B = np.asarray(B, dtype=np.int8)
    M, K = A.shape
    N = B.shape[1]
    a_sm, a_sk = _elem_strides(A)
    b_sk, b_sn = _elem_strides(B)
    zBv = _arr(np.broadcast_to(np.asarray(zB, dtype=np.int32), (N,)), np.int32)
    biasv = None if bias is None else _arr(bias, np.int32)
    out = np.zeros((M, N), dtype=np.int64)
    st = TileStats()
    rc = lib().orc_gemm_tiled(M, N, K, _ptr(A), a_sm, a_sk, int(zA), _ptr(B), b_sk, b_sn,
                              _ptr(zBv), _ptr(biasv), Tm, Tn, Tk, _ptr(out), C.byref(st))
    _check(rc, "orc_gemm_tiled")
    stats = {f: getattr(st, f) for f, _ in TileStats._fields_}
    return out, stats


# ---------------------------------------------------------------- O3
def real_multiplier(s_a, s_b, s_out):
    return lib().orc_real_multiplier(s_a, s_b, s_out)


def requant_params(real_mult):
    m0, sh = _I32(), _I32()
    rc = lib().orc_requant_params(float(real_mult), C.byref(m0), C.byref(sh))
    _check(rc, "orc_requant_params")
    return m0.value, sh.value


def rshift_rhe(t, shift):
    return lib().orc_rshift_rhe(int(t), int(shift))


def requant_value(acc, m0, shift, zp_out, lo=-128, hi=127):
    return lib().orc_requant_value(int(acc), int(m0), int(shift), int(zp_out), int(lo), int(hi))


def ideal_rhe(acc, real_mult):
    return lib().orc_ideal_rhe(int(acc), float(real_mult))


def requant_matrix(acc, s_a, s_b, s_out, zp_out, relu):
    acc = _arr(acc, np.int64)
    M, N = acc.shape
    sb = _arr(np.broadcast_to(np.asarray(s_b, dtype=np.float32), (N,)), np.float32)
    out = np.zeros((M, N), dtype=np.int8)
    nd = _I64()
    rc = lib().orc_requant_matrix(M, N, _ptr(acc), float(s_a), _ptr(sb), float(s_out),
                                  int(zp_out), int(bool(relu)), _ptr(out), C.byref(nd))
    _check(rc, "orc_requant_matrix")
    return out, nd.value


# ---------------------------------------------------------------- O5b / O6d
def quantize_rows_s8_blocked(X, block=32):
    """O5b: O5 on every block of `block` K of every row -> q, scale [M,G], zp [M,G]."""
    X = _arr(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    G = (K + block - 1) // block
    q = np.zeros((M, K), dtype=np.int8)
    sc = np.zeros((M, G), dtype=np.float32)
    zp = np.zeros((M, G), dtype=np.int32)
    lib().orc_quantize_rows_s8_blocked(M, K, block, _ptr(X), K, _ptr(q), K, _ptr(sc), _ptr(zp), G)
    return q, sc, zp


def a8w4_blockwise_blockq(qa, sa, za, qw, sw, bias, clamp_lo, clamp_hi, group=32):
    """O6d: int4 group weights x per-block quantized activations."""
    qa = _arr(qa, np.int8)
    qw = _arr(qw, np.int8)
    sw = _arr(sw, np.float32)
    sa = _arr(sa, np.float32)
    za = _arr(za, np.int32)
    M, K = qa.shape
    N = qw.shape[0]
    biasv = None if bias is None else _arr(bias, np.float32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = lib().orc_a8w4_blockwise_blockq(M, N, K, group, _ptr(qa), K, _ptr(sa), _ptr(za),
                                         sa.shape[1], _ptr(qw), K, _ptr(sw), sw.shape[1],
                                         _ptr(biasv), float(clamp_lo), float(clamp_hi), _ptr(Y), N)
    _check(rc, "orc_a8w4_blockwise_blockq")
    return Y


def a8w4_forward_blockq(X, qw, sw, bias, clamp_lo, clamp_hi, group=32):
    """Per-block dynamic quantization (O5b, blocks = the weight groups) then O6d."""
    qa, sa, za = quantize_rows_s8_blocked(X, group)
    return a8w4_blockwise_blockq(qa, sa, za, qw, sw, bias, clamp_lo, clamp_hi, group)


# ---------------------------------------------------------------- O6c
def a8w4_blockwise_asym(qa, sa, za, qw, sw, bw, bias, clamp_lo, clamp_hi, group=32):
    """O6c: asymmetric int4, w = sw*q + bw per group."""
    qa = _arr(qa, np.int8)
    qw = _arr(qw, np.int8)
    sw = _arr(sw, np.float32)
    bw = _arr(bw, np.float32)
    assert sw.shape == bw.shape
    M, K = qa.shape
    N = qw.shape[0]
    sa = _arr(sa, np.float32)
    za = _arr(za, np.int32)
    biasv = None if bias is None else _arr(bias, np.float32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = lib().orc_a8w4_blockwise_asym(M, N, K, group, _ptr(qa), K, _ptr(sa), _ptr(za), _ptr(qw),
                                       K, _ptr(sw), _ptr(bw), sw.shape[1], _ptr(biasv),
                                       float(clamp_lo), float(clamp_hi), _ptr(Y), N)
    _check(rc, "orc_a8w4_blockwise_asym")
    return Y


def a8w4_forward_asym(X, qw, sw, bw, bias, clamp_lo, clamp_hi, group=32):
    """Dynamic per-row quantization (O5) then O6c."""
    qa, sa, za = quantize_rows_s8(X)
    return a8w4_blockwise_asym(qa, sa, za, qw, sw, bw, bias, clamp_lo, clamp_hi, group)


# ---------------------------------------------------------------- O6b
def round_bf16(x):
    """O6b: f32 values rounded to the nearest bf16 (ties to even), as f32."""
    x = _arr(np.asarray(x, np.float32), np.float32)
    y = np.zeros_like(x)
    lib().orc_round_bf16_array(x.size, _ptr(x), _ptr(y))
    return y


# ---------------------------------------------------------------- O9
def dequant_weights_s8(W_nk, s, z):
    """O9 (int8): f32 sB[n]*(q[n,k] - zB[n]), one IEEE f32 product per value
    ([TRACT] extract_at_mn_f32 returns packed values as floats; the scale
    and zero point are those stored beside the weights)."""
    W = np.asarray(W_nk).astype(np.int32)
    N = W.shape[0]
    sv = np.broadcast_to(np.asarray(s, np.float32), (N,))
    zv = np.broadcast_to(np.asarray(z, np.int32), (N,))
    return sv[:, None] * (W - zv[:, None]).astype(np.float32)


def dequant_weights_s4(W_nk, sw, group=32, bw=None):
    """O9 (int4): f32 sw[n, k // group]*q[n,k], one IEEE f32 product per value;
    asymmetric weights (O6c) then add the group offset in f32."""
    W = np.asarray(W_nk).astype(np.float32)
    sw = np.asarray(sw, np.float32)
    g = np.arange(W.shape[1]) // group
    y = sw[:, g] * W
    if bw is not None:
        y = y + np.asarray(bw, np.float32)[:, g]
    return y


# ---------------------------------------------------------------- O8
def dequant_matrix_f32(acc, s_a, s_b, bias, lo, hi):
    """O8: Y = f32(clamp(sA*sB[n]*acc + bias[n], lo, hi)), in fp64."""
    acc = _arr(acc, np.int64)
    M, N = acc.shape
    sb = _arr(np.broadcast_to(np.asarray(s_b, dtype=np.float32), (N,)), np.float32)
    bv = None if bias is None else _arr(bias, np.float32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = lib().orc_dequant_matrix_f32(M, N, _ptr(acc), float(s_a), _ptr(sb), _ptr(bv),
                                      float(lo), float(hi), _ptr(Y))
    _check(rc, "orc_dequant_matrix_f32")
    return Y


# ---------------------------------------------------------------- O4
def conv_out_dims(H, W, KH, KW, stride=(1, 1), pad=(0, 0, 0, 0), dilation=(1, 1)):
    OH = (H + pad[0] + pad[2] - (dilation[0] * (KH - 1) + 1)) // stride[0] + 1
    OW = (W + pad[1] + pad[3] - (dilation[1] * (KW - 1) + 1)) // stride[1] + 1
    return OH, OW


def conv2d_direct(X, zp_in, Wt, stride=(1, 1), pad=(0, 0, 0, 0), bias=None, dilation=(1, 1)):
    """X: int8 NHWC; Wt: int8 OIHW; pad = (top, left, bottom, right)."""
    X = _arr(X, np.int8)
    Wt = _arr(Wt, np.int8)
    NB, H, W, Cc = X.shape
    OC, IC, KH, KW = Wt.shape
    assert IC == Cc
    OH, OW = conv_out_dims(H, W, KH, KW, stride, pad, dilation)
    out = np.zeros((NB, OH, OW, OC), dtype=np.int64)
    biasv = None if bias is None else _arr(bias, np.int32)
    rc = lib().orc_conv2d_direct(NB, H, W, Cc, _ptr(X), int(zp_in), OC, KH, KW, _ptr(Wt),
                                 stride[0], stride[1], pad[0], pad[1], pad[2], pad[3],
                                 dilation[0], dilation[1], _ptr(biasv), _ptr(out))
    _check(rc, "orc_conv2d_direct")
    return out


def conv2d_blockwise_f32(X, zx, sx, Wt, icb, sw, stride=(1, 1), pad=(0, 0, 0, 0), bias=None,
                         dilation=(1, 1), lo=-np.inf, hi=np.inf):
    """O4c: conv with per-(oc, input-channel block) weight scales, f32 out."""
    X = _arr(X, np.int8)
    Wt = _arr(Wt, np.int8)
    NB, H, W, Cc = X.shape
    OC, IC, KH, KW = Wt.shape
    assert IC == Cc
    OH, OW = conv_out_dims(H, W, KH, KW, stride, pad, dilation)
    swv = _arr(sw, np.float32)
    biasv = None if bias is None else _arr(bias, np.float32)
    Y = np.zeros((NB, OH, OW, OC), dtype=np.float32)
    rc = lib().orc_conv2d_blockwise_f32(NB, H, W, Cc, _ptr(X), int(zx), float(sx), OC, KH, KW,
                                        _ptr(Wt), stride[0], stride[1], pad[0], pad[1], pad[2],
                                        pad[3], dilation[0], dilation[1], icb, _ptr(swv),
                                        _ptr(biasv), float(lo), float(hi), _ptr(Y))
    _check(rc, "orc_conv2d_blockwise_f32")
    return Y


def im2col(X, pad_value, KH, KW, stride=(1, 1), pad=(0, 0, 0, 0), dilation=(1, 1)):
    X = _arr(X, np.int8)
    NB, H, W, Cc = X.shape
    OH, OW = conv_out_dims(H, W, KH, KW, stride, pad, dilation)
    col = np.zeros((NB * OH * OW, KH * KW * Cc), dtype=np.int8)
    rc = lib().orc_im2col(NB, H, W, Cc, _ptr(X), int(pad_value), KH, KW, stride[0], stride[1],
                          pad[0], pad[1], pad[2], pad[3], dilation[0], dilation[1], _ptr(col))
    _check(rc, "orc_im2col")
    return col


# ---------------------------------------------------------------- O5
def quantize_rows_s8(X):
    X = _arr(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    q = np.zeros((M, K), dtype=np.int8)
    sc = np.zeros(M, dtype=np.float32)
    zp = np.zeros(M, dtype=np.int32)
    lib().orc_quantize_rows_s8(M, K, _ptr(X), K, _ptr(q), K, _ptr(sc), _ptr(zp))
    return q, sc, zp


def quantize_rows_s8_sym(X):
    """O5s: symmetric per-row quantization; returns (q, scale)."""
    X = _arr(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    q = np.zeros((M, K), dtype=np.int8)
    sc = np.zeros(M, dtype=np.float32)
    lib().orc_quantize_rows_s8_sym(M, K, _ptr(X), K, _ptr(q), K, _ptr(sc))
    return q, sc


# ---------------------------------------------------------------- O6
def a8w4_blockwise(qa, sa, za, qw, sw, bias, clamp_lo, clamp_hi, group=32):
    qa = _arr(qa, np.int8)
    qw = _arr(qw, np.int8)
    sw = _arr(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    sa = _arr(sa, np.float32)
    za = _arr(za, np.int32)
    biasv = None if bias is None else _arr(bias, np.float32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = lib().orc_a8w4_blockwise(M, N, K, group, _ptr(qa), K, _ptr(sa), _ptr(za), _ptr(qw), K,
                                  _ptr(sw), sw.shape[1], _ptr(biasv), float(clamp_lo),
                                  float(clamp_hi), _ptr(Y), N)
    _check(rc, "orc_a8w4_blockwise")
    return Y


def a8w4_forward(X, qw, sw, bias, clamp_lo, clamp_hi, group=32):
    """The whole A8W4 path: dynamic per-row quantization (O5) then O6."""
    qa, sa, za = quantize_rows_s8(X)
    return a8w4_blockwise(qa, sa, za, qw, sw, bias, clamp_lo, clamp_hi, group)


# ---------------------------------------------------------------- O7
def pack_s8_ref(W_nk, scales, zps=None, per_channel=True):
    """Reference blob for int8 weights given as a logical [N,K] array (any strides)."""
    W_nk = np.asarray(W_nk, dtype=np.int8)
    N, K = W_nk.shape
    w_sn, w_sk = _elem_strides(W_nk)
    sc = _arr(scales, np.float32)
    zpv = None if zps is None else _arr(zps, np.int32)
    nbytes = lib().orc_packed_s8_bytes(N, K)
    blob = np.zeros(nbytes, dtype=np.uint8)
    rc = lib().orc_pack_s8_ref(N, K, _ptr(W_nk), w_sn, w_sk, int(bool(per_channel)), _ptr(sc),
                               _ptr(zpv), _ptr(blob))
    _check(rc, "orc_pack_s8_ref")
    return blob


def pack_s4_ref(W_nk, sw, group=32):
    W_nk = np.asarray(W_nk, dtype=np.int8)
    N, K = W_nk.shape
    w_sn, w_sk = _elem_strides(W_nk)
    sw = _arr(sw, np.float32)
    nbytes = lib().orc_packed_s4_bytes(N, K, group)
    if nbytes < 0:
        raise OracleError("unsupported group %d" % group)
    blob = np.zeros(nbytes, dtype=np.uint8)
    rc = lib().orc_pack_s4_ref(N, K, group, _ptr(W_nk), w_sn, w_sk, _ptr(sw), sw.shape[1],
                               _ptr(blob))
    _check(rc, "orc_pack_s4_ref")
    return blob
