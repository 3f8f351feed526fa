"""Python binding of ``libqpack.so``, the gfx950 quantized integer matmul.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The functions carry
the C ABI's names (see ``include/qpack.h`` for the contract of each).  If the
shared library is missing this module raises at import -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqpack.so")

QP_OK, QP_EINVAL, QP_EUNSUPPORTED, QP_EOVERFLOW, QP_ESIZE, QP_EALIGN, QP_EHIP = 0, -1, -2, -3, -4, -5, -6
QP_S8, QP_S4, QP_S32, QP_F32 = 1, 2, 3, 4
QP_PER_TENSOR, QP_PER_CHANNEL, QP_BLOCKWISE, QP_DYNAMIC_PER_ROW = 0, 1, 2, 3
QP_BLOCKWISE_BF16, QP_BLOCKWISE_ASYM = 4, 5
QP_ROUND_HALF_EVEN = 0

_STATUS = {0: "QP_OK", -1: "QP_EINVAL", -2: "QP_EUNSUPPORTED", -3: "QP_EOVERFLOW",
           -4: "QP_ESIZE", -5: "QP_EALIGN", -6: "QP_EHIP"}


class QTensor(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("rank", C.c_int32), ("shape", C.c_int64 * 4),
                ("stride", C.c_int64 * 4), ("scheme", C.c_int32), ("axis", C.c_int32),
                ("group_size", C.c_int32), ("scale", C.c_float), ("scales", C.c_void_p),
                ("zero_point", C.c_int32), ("zero_points", C.c_void_p), ("qmin", C.c_int32),
                ("qmax", C.c_int32), ("rounding", C.c_int32)]


class PackedInfo(C.Structure):
    _fields_ = [("format", C.c_int32), ("scheme", C.c_int32), ("N", C.c_int64), ("K", C.c_int64),
                ("Npad", C.c_int64), ("Kpad", C.c_int64), ("group", C.c_int64),
                ("data_off", C.c_int64), ("data_bytes", C.c_int64), ("scale_off", C.c_int64),
                ("sum_off", C.c_int64), ("zp_off", C.c_int64), ("total_bytes", C.c_int64),
                ("has_zero_points", C.c_int32), ("scale_min", C.c_float), ("scale_max", C.c_float)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class QPackError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (_STATUS.get(status, "?"), status, msg))
        self.status = status


_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_F = C.c_float
_QT = C.POINTER(QTensor)
_PI = C.POINTER(PackedInfo)
_SZ = C.POINTER(C.c_size_t)

SIGNATURES = {
    "qp_version": (C.c_char_p, []),
    "qp_last_error": (C.c_char_p, []),
    "qpack_weights_size": (C.c_int, [_QT, _I32, _I32, _SZ, _SZ]),
    "qpack_weights": (C.c_int, [_QT, _P, _I32, _I32, _P, C.c_size_t, _PI, _P]),
    "qrepack_weights": (C.c_int, [_QT, _P, _I32, _I32, _P, _PI, _P]),
    "qp_packed_info_from_header": (C.c_int, [_P, _PI]),
    "qunpack_weights": (C.c_int, [_PI, _P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P]),
    "qquantize_rows_s8": (C.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _P]),
    "qquantize_rows_s8_sym": (C.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "qgemm_s8s8_requant_ws_size": (C.c_int, [_QT, _PI, _SZ]),
    "qgemm_s8s8_requant": (C.c_int, [_QT, _P, _PI, _P, _P, _I64, _QT, _I32, _P, _P, C.c_size_t,
                                     _P]),
    "qgemm_s8s8_dequant_f32": (C.c_int, [_QT, _P, _PI, _P, _P, _F, _F, _P, _I64, _P,
                                         C.c_size_t, _P]),
    "qquantize_rows_s8_blocked": (C.c_int, [_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P, _P,
                                            _I64, _P]),
    "qgemm_a8w4_blockq_f32_ws_size": (C.c_int, [_I64, _PI, _SZ]),
    "qgemm_a8w4_blockq_f32": (C.c_int, [_P, _I64, _I64, _I64, _PI, _P, _P, _F, _F, _P, _I64, _P,
                                        C.c_size_t, _P]),
    "qgemm_a8w4_blockq_prequant_f32": (C.c_int, [_P, _I64, _I64, _P, _P, _I64, _PI, _P, _P, _F,
                                                 _F, _P, _I64, _P]),
    "qgemm_a8w8_blockwise_f32_ws_size": (C.c_int, [_I64, _PI, _SZ]),
    "qgemm_a8w8_blockwise_f32": (C.c_int, [_P, _I64, _I64, _I64, _PI, _P, _P, _F, _F, _P, _I64,
                                           _P, C.c_size_t, _P]),
    "qgemm_a8w8_blockwise_prequant_f32": (C.c_int, [_P, _I64, _I64, _P, _P, _PI, _P, _P, _F, _F,
                                                    _P, _I64, _P]),
    "qgemm_a8w4_blockwise_f32_ws_size": (C.c_int, [_I64, _PI, _SZ]),
    "qgemm_a8w4_blockwise_f32": (C.c_int, [_P, _I64, _I64, _I64, _PI, _P, _P, _F, _F, _P, _I64,
                                           _P, C.c_size_t, _P]),
    "qgemm_a8w4_prequant_f32": (C.c_int, [_P, _I64, _I64, _P, _P, _PI, _P, _P, _F, _F, _P, _I64,
                                          _P]),
    "qgemm_a8w4_blockwise_f32_noalloc": (C.c_int, [_P, _I64, _I64, _I64, _PI, _P, _P, _F, _F, _P,
                                                   _I64, _P]),
    "qim2col_s8": (C.c_int, [_P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32,
                             _I32, _I32, _I32, _P, _I64, _P]),
    "qconv2d_s8_im2col_ws_size": (C.c_int, [_QT, _PI, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                            _I32, _SZ]),
    "qconv2d_s8_im2col": (C.c_int, [_QT, _P, _PI, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                    _I32, _P, _I64, _QT, _I32, _P, _P, C.c_size_t, _P]),
    "qconv2d_s8_blockwise_f32": (C.c_int, [_QT, _P, _PI, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, _P, _F, _F, _P, _P]),
    "qconv2d_s8_ws_size": (C.c_int, [_QT, _PI, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                     _I32, _I32, _SZ]),
    "qconv2d_s8": (C.c_int, [_QT, _P, _PI, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                             _I32, _I32, _P, _I64, _QT, _I32, _P, _P, C.c_size_t, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqpack.so is not built (expected at %s); run "
                          "`python conv_qpack_weights_amd/build.py`" % LIB_PATH)
    h = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(h, name)
        f.restype = res
        f.argtypes = args
    return h


_lib = _load()


def lib():
    return _lib


def last_error() -> str:
    return (_lib.qp_last_error() or b"").decode()


def _check(status, what=""):
    if status != QP_OK:
        raise QPackError(status, "%s: %s" % (what, last_error()))


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def qtensor(dtype, shape, stride=None, scheme=QP_PER_TENSOR, scale=1.0, scales=None,
            zero_point=0, zero_points=None, axis=0, group_size=0, qmin=-128, qmax=127,
            rounding=QP_ROUND_HALF_EVEN) -> QTensor:
    """Build a qp_qtensor descriptor (``scales``/``zero_points``: device tensors or None)."""
    q = QTensor()
    q.dtype = dtype
    q.rank = len(shape)
    if stride is None:
        stride, acc = [], 1
        for d in reversed(shape):
            stride.insert(0, acc)
            acc *= d
    for i, (d, s) in enumerate(zip(shape, stride)):
        q.shape[i] = int(d)
        q.stride[i] = int(s)
    q.scheme = scheme
    q.axis = axis
    q.group_size = group_size
    q.scale = float(scale)
    q.scales = None if scales is None else scales.data_ptr()
    q.zero_point = int(zero_point)
    q.zero_points = None if zero_points is None else zero_points.data_ptr()
    q.qmin, q.qmax, q.rounding = qmin, qmax, rounding
    return q


def _alloc_bytes(n, device):
    # torch's caching allocator returns at least 256-byte aligned blocks
    t = torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


# ---------------------------------------------------------------- packing
def qpack_weights_size(desc: QTensor, k_axis: int, n_axis: int):
    nb, al = C.c_size_t(), C.c_size_t()
    _check(_lib.qpack_weights_size(C.byref(desc), k_axis, n_axis, C.byref(nb), C.byref(al)),
           "qpack_weights_size")
    return nb.value, al.value


def qpack_weights(w: torch.Tensor, desc: QTensor, k_axis: int, n_axis: int, into=None):
    """Pack device weights ``w`` described by ``desc``; returns (blob, PackedInfo).
    ``into=(blob, info)``: refill that existing blob in place instead
    (qrepack_weights; same shape and format required), returning it."""
    if into is not None:
        blob, info = into
        _check(_lib.qrepack_weights(C.byref(desc), _ptr(w), k_axis, n_axis, _ptr(blob),
                                    C.byref(info), _stream(w.device)), "qrepack_weights")
        return blob, info
    nbytes, _ = qpack_weights_size(desc, k_axis, n_axis)
    blob = _alloc_bytes(nbytes, w.device)
    info = PackedInfo()
    _check(_lib.qpack_weights(C.byref(desc), _ptr(w), k_axis, n_axis, _ptr(blob), nbytes,
                              C.byref(info), _stream(w.device)), "qpack_weights")
    return blob, info


def pack_s8(w: torch.Tensor, scales=None, scale=1.0, zero_points=None, zero_point=0,
            k_axis=None, n_axis=None, into=None):
    """Pack int8 weights: rank 2 ([N,K] by default) or rank 4 OIHW.
    ``into=(blob, info)`` refills an existing blob of the same shape."""
    if w.dim() == 4:
        k_axis, n_axis = 1, 0
    elif k_axis is None:
        k_axis, n_axis = 1, 0
    scheme = QP_PER_CHANNEL if scales is not None else QP_PER_TENSOR
    desc = qtensor(QP_S8, list(w.shape), [s for s in w.stride()], scheme=scheme, scale=scale,
                   scales=scales, zero_point=zero_point, zero_points=zero_points, axis=n_axis)
    return qpack_weights(w, desc, k_axis, n_axis, into)


def pack_s8_blockwise(w: torch.Tensor, scales: torch.Tensor, block=128, into=None):
    """Pack int8 weights with one f32 scale per channel and block: rank 2
    [N, K] with scales [N, ceil(K/block)] (blocks of K), or OIHW with scales
    [OC, IC/block] (blocks of input channels, every kernel tap)."""
    k_axis, n_axis = 1, 0
    desc = qtensor(QP_S8, list(w.shape), list(w.stride()), scheme=QP_BLOCKWISE, scales=scales,
                   group_size=block, axis=n_axis)
    return qpack_weights(w, desc, k_axis, n_axis, into)


def pack_s4(w: torch.Tensor, scales: torch.Tensor, group_size=32, scale_dtype="f32",
            offsets=None, into=None):
    """Pack int4 values (one per int8 byte, in [-8,7]) given as [N, K] with
    f32 group scales [N, ceil(K/group)]; scale_dtype "bf16" stores the
    scales rounded to bf16; `offsets` [N, ceil(K/group)] makes the weights
    asymmetric (real weight = scale*q + offset).  ``into=(blob, info)``
    refills an existing blob of the same shape and format."""
    scheme = {"f32": QP_BLOCKWISE, "bf16": QP_BLOCKWISE_BF16}[scale_dtype]
    if offsets is not None:
        assert scale_dtype == "f32", "asymmetric int4 keeps f32 scales"
        scheme = QP_BLOCKWISE_ASYM
        scales = torch.stack((offsets.float(), scales.float()), dim=-1).contiguous()
    desc = qtensor(QP_S4, list(w.shape), list(w.stride()), scheme=scheme, scales=scales,
                   group_size=group_size, axis=0)
    return qpack_weights(w, desc, 1, 0, into)


def qp_packed_info_from_header(header: bytes) -> PackedInfo:
    info = PackedInfo()
    buf = C.create_string_buffer(bytes(header), 256)
    _check(_lib.qp_packed_info_from_header(buf, C.byref(info)), "qp_packed_info_from_header")
    return info


def qunpack_weights(blob: torch.Tensor, info: PackedInfo, n_begin=0, n_count=None,
                    values=True, scales=True, dequant=False):
    """Channels [n_begin, n_begin+n_count) of a blob as logical int8 values
    [n, K], their scales (int8 blob: [n]; int4: [n, groups]), zero points
    (int8 blob) and optionally the dequantized f32 weights [n, K]."""
    n_count = info.N - n_begin if n_count is None else n_count
    dev = blob.device
    K = info.K
    groups = 1 if info.format == 1 else (K + info.group - 1) // info.group
    if info.format == 4:
        groups *= 2   # (offset, scale) pairs
    w = torch.empty((n_count, K), dtype=torch.int8, device=dev) if values else None
    sc = None
    if scales:
        sc = torch.empty((n_count,) if info.format == 1 else (n_count, groups),
                         dtype=torch.float32, device=dev)
    zp = torch.empty(n_count, dtype=torch.int32, device=dev) if (scales and info.format == 1) \
        else None
    dq = torch.empty((n_count, K), dtype=torch.float32, device=dev) if dequant else None
    _check(_lib.qunpack_weights(C.byref(info), _ptr(blob), n_begin, n_count, _ptr(w), K, _ptr(sc),
                                groups, _ptr(zp), _ptr(dq), K, _stream(dev)), "qunpack_weights")
    return w, sc, zp, dq


def blob_to_bytes(blob: torch.Tensor) -> bytes:
    """The blob as bytes (it describes itself: header, then the regions)."""
    return blob.cpu().numpy().tobytes()


def blob_from_bytes(data: bytes, device="cuda"):
    """A blob restored from bytes onto `device`, with its info decoded (and
    validated) from the header."""
    info = qp_packed_info_from_header(data[:256])
    if len(data) < info.total_bytes:
        raise QPackError(QP_ESIZE, "blob bytes: %d, header says %d"
                         % (len(data), info.total_bytes))
    blob = _alloc_bytes(info.total_bytes, device)
    blob.copy_(torch.frombuffer(bytearray(data[:info.total_bytes]), dtype=torch.uint8))
    return blob, info


# ---------------------------------------------------------------- quantizer
def qquantize_rows_s8(x: torch.Tensor, q=None, row_scale=None, row_zp=None):
    assert x.dim() == 2 and x.dtype == torch.float32 and x.stride(1) == 1
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    row_scale = torch.empty(M, dtype=torch.float32, device=x.device) if row_scale is None else row_scale
    row_zp = torch.empty(M, dtype=torch.int32, device=x.device) if row_zp is None else row_zp
    _check(_lib.qquantize_rows_s8(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0),
                                  _ptr(row_scale), _ptr(row_zp), _stream(x.device)),
           "qquantize_rows_s8")
    return q, row_scale, row_zp


def qquantize_rows_s8_sym(x: torch.Tensor, q=None, row_scale=None):
    assert x.dim() == 2 and x.dtype == torch.float32 and x.stride(1) == 1
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    row_scale = torch.empty(M, dtype=torch.float32, device=x.device) if row_scale is None else row_scale
    _check(_lib.qquantize_rows_s8_sym(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0),
                                      _ptr(row_scale), _stream(x.device)),
           "qquantize_rows_s8_sym")
    return q, row_scale


# ---------------------------------------------------------------- int8 GEMM
def qgemm_s8s8_requant_ws_size(a_desc: QTensor, info: PackedInfo) -> int:
    n = C.c_size_t()
    _check(_lib.qgemm_s8s8_requant_ws_size(C.byref(a_desc), C.byref(info), C.byref(n)),
           "qgemm_s8s8_requant_ws_size")
    return n.value


def qgemm_s8s8_requant(A: torch.Tensor, sA: float, zA: int, blob: torch.Tensor, info: PackedInfo,
                       bias=None, max_abs_bias=0, s_out=1.0, zp_out=0, relu=False,
                       out_dtype="s8", out=None, ws=None):
    """C[M,N] = requant(A @ B + bias) (int8) or the corrected INT32 accumulator."""
    assert A.dtype == torch.int8 and A.dim() == 2 and A.stride(1) == 1
    M, K = A.shape
    a_desc = qtensor(QP_S8, [M, K], [A.stride(0), 1], scale=sA, zero_point=zA)
    tdt = torch.int8 if out_dtype == "s8" else torch.int32
    if out is None:
        out = torch.empty((M, info.N), dtype=tdt, device=A.device)
    o_desc = qtensor(QP_S8 if out_dtype == "s8" else QP_S32, [M, info.N], [out.stride(0), 1],
                     scale=s_out, zero_point=zp_out)
    if ws is None:
        ws = _alloc_bytes(qgemm_s8s8_requant_ws_size(a_desc, info), A.device)
    _check(_lib.qgemm_s8s8_requant(C.byref(a_desc), _ptr(A), C.byref(info), _ptr(blob),
                                   _ptr(bias), int(max_abs_bias), C.byref(o_desc), int(bool(relu)),
                                   _ptr(out), _ptr(ws), ws.numel(), _stream(A.device)),
           "qgemm_s8s8_requant")
    return out


def qgemm_s8s8_dequant_f32(A: torch.Tensor, sA: float, zA: int, blob: torch.Tensor,
                           info: PackedInfo, bias=None, clamp_lo=-float("inf"),
                           clamp_hi=float("inf"), out=None, ws=None):
    """Y[M,N] = clamp(sA*sB[n]*(A-zA)@(B-zB) + bias, lo, hi) in f32."""
    assert A.dtype == torch.int8 and A.dim() == 2 and A.stride(1) == 1
    M, K = A.shape
    a_desc = qtensor(QP_S8, [M, K], [A.stride(0), 1], scale=sA, zero_point=zA)
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=A.device)
    assert out.dtype == torch.float32 and out.stride(1) == 1
    if ws is None:
        ws = _alloc_bytes(qgemm_s8s8_requant_ws_size(a_desc, info), A.device)
    _check(_lib.qgemm_s8s8_dequant_f32(C.byref(a_desc), _ptr(A), C.byref(info), _ptr(blob),
                                       _ptr(bias), clamp_lo, clamp_hi, _ptr(out), out.stride(0),
                                       _ptr(ws), ws.numel(), _stream(A.device)),
           "qgemm_s8s8_dequant_f32")
    return out


# ---------------------------------------------------------------- A8W4
def qgemm_a8w4_blockwise_f32_ws_size(M: int, info: PackedInfo) -> int:
    n = C.c_size_t()
    _check(_lib.qgemm_a8w4_blockwise_f32_ws_size(M, C.byref(info), C.byref(n)),
           "qgemm_a8w4_blockwise_f32_ws_size")
    return n.value


def qgemm_a8w4_blockwise_f32(X: torch.Tensor, blob: torch.Tensor, info: PackedInfo, bias=None,
                             clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None, ws=None):
    assert X.dtype == torch.float32 and X.dim() == 2 and X.stride(1) == 1
    M, K = X.shape
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = _alloc_bytes(qgemm_a8w4_blockwise_f32_ws_size(M, info), X.device)
    _check(_lib.qgemm_a8w4_blockwise_f32(_ptr(X), M, K, X.stride(0), C.byref(info), _ptr(blob),
                                         _ptr(bias), clamp_lo, clamp_hi, _ptr(out), out.stride(0),
                                         _ptr(ws), ws.numel(), _stream(X.device)),
           "qgemm_a8w4_blockwise_f32")
    return out


def qgemm_a8w4_blockwise_f32_noalloc(X: torch.Tensor, blob: torch.Tensor, info: PackedInfo,
                                     bias=None, clamp_lo=-float("inf"), clamp_hi=float("inf"),
                                     out=None):
    """qgemm_a8w4_blockwise_f32 without a workspace: the library's own
    per-GPU scratch array holds the quantized rows (at most 4 MiB)."""
    assert X.dtype == torch.float32 and X.dim() == 2 and X.stride(1) == 1
    M, K = X.shape
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=X.device)
    _check(_lib.qgemm_a8w4_blockwise_f32_noalloc(_ptr(X), M, K, X.stride(0), C.byref(info),
                                                 _ptr(blob), _ptr(bias), clamp_lo, clamp_hi,
                                                 _ptr(out), out.stride(0), _stream(X.device)),
           "qgemm_a8w4_blockwise_f32_noalloc")
    return out


def qgemm_a8w4_prequant_f32(qa: torch.Tensor, sa: torch.Tensor, za: torch.Tensor,
                            blob: torch.Tensor, info: PackedInfo, bias=None,
                            clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None):
    M = qa.shape[0]
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=qa.device)
    _check(_lib.qgemm_a8w4_prequant_f32(_ptr(qa), M, qa.stride(0), _ptr(sa), _ptr(za),
                                        C.byref(info), _ptr(blob), _ptr(bias), clamp_lo, clamp_hi,
                                        _ptr(out), out.stride(0), _stream(qa.device)),
           "qgemm_a8w4_prequant_f32")
    return out


def qquantize_rows_s8_blocked(x: torch.Tensor, block=32, kpad=None, q=None, scale=None,
                              zp=None):
    """Per-(row, block of 32) dynamic quantization: q [M, kpad], scale and zp
    [M, kpad/32]."""
    assert x.dim() == 2 and x.dtype == torch.float32 and x.stride(1) == 1
    M, K = x.shape
    kpad = ((K + 31) // 32) * 32 if kpad is None else kpad
    nb = kpad // 32
    q = torch.empty((M, kpad), dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty((M, nb), dtype=torch.float32, device=x.device) if scale is None else scale
    zp = torch.empty((M, nb), dtype=torch.int32, device=x.device) if zp is None else zp
    _check(_lib.qquantize_rows_s8_blocked(_ptr(x), M, K, x.stride(0), block, kpad, _ptr(q),
                                          q.stride(0), _ptr(scale), _ptr(zp), scale.stride(0),
                                          _stream(x.device)), "qquantize_rows_s8_blocked")
    return q, scale, zp


def qgemm_a8w4_blockq_f32_ws_size(M: int, info: PackedInfo) -> int:
    n = C.c_size_t()
    _check(_lib.qgemm_a8w4_blockq_f32_ws_size(M, C.byref(info), C.byref(n)),
           "qgemm_a8w4_blockq_f32_ws_size")
    return n.value


def qgemm_a8w4_blockq_f32(X: torch.Tensor, blob: torch.Tensor, info: PackedInfo, bias=None,
                          clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None, ws=None):
    assert X.dtype == torch.float32 and X.dim() == 2 and X.stride(1) == 1
    M, K = X.shape
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = _alloc_bytes(qgemm_a8w4_blockq_f32_ws_size(M, info), X.device)
    _check(_lib.qgemm_a8w4_blockq_f32(_ptr(X), M, K, X.stride(0), C.byref(info), _ptr(blob),
                                      _ptr(bias), clamp_lo, clamp_hi, _ptr(out), out.stride(0),
                                      _ptr(ws), ws.numel(), _stream(X.device)),
           "qgemm_a8w4_blockq_f32")
    return out


def qgemm_a8w4_blockq_prequant_f32(qa: torch.Tensor, sa: torch.Tensor, za: torch.Tensor,
                                   blob: torch.Tensor, info: PackedInfo, bias=None,
                                   clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None):
    M = qa.shape[0]
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=qa.device)
    _check(_lib.qgemm_a8w4_blockq_prequant_f32(_ptr(qa), M, qa.stride(0), _ptr(sa), _ptr(za),
                                               sa.stride(0), C.byref(info), _ptr(blob),
                                               _ptr(bias), clamp_lo, clamp_hi, _ptr(out),
                                               out.stride(0), _stream(qa.device)),
           "qgemm_a8w4_blockq_prequant_f32")
    return out


def qgemm_a8w8_blockwise_f32_ws_size(M: int, info: PackedInfo) -> int:
    n = C.c_size_t()
    _check(_lib.qgemm_a8w8_blockwise_f32_ws_size(M, C.byref(info), C.byref(n)),
           "qgemm_a8w8_blockwise_f32_ws_size")
    return n.value


def qgemm_a8w8_blockwise_f32(X: torch.Tensor, blob: torch.Tensor, info: PackedInfo, bias=None,
                             clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None, ws=None):
    assert X.dtype == torch.float32 and X.dim() == 2 and X.stride(1) == 1
    M, K = X.shape
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = _alloc_bytes(qgemm_a8w8_blockwise_f32_ws_size(M, info), X.device)
    _check(_lib.qgemm_a8w8_blockwise_f32(_ptr(X), M, K, X.stride(0), C.byref(info), _ptr(blob),
                                         _ptr(bias), clamp_lo, clamp_hi, _ptr(out), out.stride(0),
                                         _ptr(ws), ws.numel(), _stream(X.device)),
           "qgemm_a8w8_blockwise_f32")
    return out


def qgemm_a8w8_blockwise_prequant_f32(qa: torch.Tensor, sa: torch.Tensor, za: torch.Tensor,
                                      blob: torch.Tensor, info: PackedInfo, bias=None,
                                      clamp_lo=-float("inf"), clamp_hi=float("inf"), out=None):
    M = qa.shape[0]
    if out is None:
        out = torch.empty((M, info.N), dtype=torch.float32, device=qa.device)
    _check(_lib.qgemm_a8w8_blockwise_prequant_f32(_ptr(qa), M, qa.stride(0), _ptr(sa), _ptr(za),
                                                  C.byref(info), _ptr(blob), _ptr(bias),
                                                  clamp_lo, clamp_hi, _ptr(out), out.stride(0),
                                                  _stream(qa.device)),
           "qgemm_a8w8_blockwise_prequant_f32")
    return out


# ---------------------------------------------------------------- conv
def qim2col_s8(X: torch.Tensor, pad_value: int, KH: int, KW: int, stride=(1, 1),
               pad=(0, 0, 0, 0), ldcol=None):
    NB, H, W, Cc = X.shape
    OH = (H + pad[0] + pad[2] - KH) // stride[0] + 1
    OW = (W + pad[1] + pad[3] - KW) // stride[1] + 1
    K = KH * KW * Cc
    ldcol = ldcol or ((K + 15) // 16) * 16
    col = torch.empty((NB * OH * OW, ldcol), dtype=torch.int8, device=X.device)
    _check(_lib.qim2col_s8(_ptr(X), NB, H, W, Cc, int(pad_value), KH, KW, stride[0], stride[1],
                           pad[0], pad[1], pad[2], pad[3], _ptr(col), ldcol, _stream(X.device)),
           "qim2col_s8")
    return col


def qconv2d_s8_im2col(X: torch.Tensor, s_in: float, zp_in: int, blob: torch.Tensor,
                      info: PackedInfo, KH: int, KW: int, stride=(1, 1), pad=(0, 0, 0, 0),
                      bias=None, max_abs_bias=0, s_out=1.0, zp_out=0, relu=False,
                      out_dtype="s8", out=None, ws=None):
    NB, H, W, Cc = X.shape
    OH = (H + pad[0] + pad[2] - KH) // stride[0] + 1
    OW = (W + pad[1] + pad[3] - KW) // stride[1] + 1
    x_desc = qtensor(QP_S8, [NB, H, W, Cc], scale=s_in, zero_point=zp_in)
    tdt = torch.int8 if out_dtype == "s8" else torch.int32
    if out is None:
        out = torch.empty((NB, OH, OW, info.N), dtype=tdt, device=X.device)
    y_desc = qtensor(QP_S8 if out_dtype == "s8" else QP_S32, [NB, OH, OW, info.N], scale=s_out,
                     zero_point=zp_out)
    if ws is None:
        n = C.c_size_t()
        _check(_lib.qconv2d_s8_im2col_ws_size(C.byref(x_desc), C.byref(info), KH, KW, stride[0],
                                              stride[1], pad[0], pad[1], pad[2], pad[3],
                                              C.byref(n)), "qconv2d_s8_im2col_ws_size")
        ws = _alloc_bytes(n.value, X.device)
    _check(_lib.qconv2d_s8_im2col(C.byref(x_desc), _ptr(X), C.byref(info), _ptr(blob), KH, KW,
                                  stride[0], stride[1], pad[0], pad[1], pad[2], pad[3],
                                  _ptr(bias), int(max_abs_bias), C.byref(y_desc), int(bool(relu)),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(X.device)),
           "qconv2d_s8_im2col")
    return out


def qconv2d_s8(X: torch.Tensor, s_in: float, zp_in: int, blob: torch.Tensor, info: PackedInfo,
               KH: int, KW: int, stride=(1, 1), pad=(0, 0, 0, 0), dilation=(1, 1), bias=None,
               max_abs_bias=0, s_out=1.0, zp_out=0, relu=False, out_dtype="s8", out=None,
               ws=None):
    """General INT8 NHWC convolution: implicit GEMM when C % 16 == 0, the GEMM
    itself for a 1x1/stride-1/unpadded kernel, explicit im2col otherwise."""
    NB, H, W, Cc = X.shape
    OH = (H + pad[0] + pad[2] - (dilation[0] * (KH - 1) + 1)) // stride[0] + 1
    OW = (W + pad[1] + pad[3] - (dilation[1] * (KW - 1) + 1)) // stride[1] + 1
    x_desc = qtensor(QP_S8, [NB, H, W, Cc], scale=s_in, zero_point=zp_in)
    tdt = torch.int8 if out_dtype == "s8" else torch.int32
    if out is None:
        out = torch.empty((NB, OH, OW, info.N), dtype=tdt, device=X.device)
    y_desc = qtensor(QP_S8 if out_dtype == "s8" else QP_S32, [NB, OH, OW, info.N], scale=s_out,
                     zero_point=zp_out)
    geom = (KH, KW, stride[0], stride[1], pad[0], pad[1], pad[2], pad[3], dilation[0],
            dilation[1])
    if ws is None:
        n = C.c_size_t()
        _check(_lib.qconv2d_s8_ws_size(C.byref(x_desc), C.byref(info), *geom, C.byref(n)),
               "qconv2d_s8_ws_size")
        ws = _alloc_bytes(n.value, X.device)
    _check(_lib.qconv2d_s8(C.byref(x_desc), _ptr(X), C.byref(info), _ptr(blob), *geom,
                           _ptr(bias), int(max_abs_bias), C.byref(y_desc), int(bool(relu)),
                           _ptr(out), _ptr(ws), ws.numel(), _stream(X.device)),
           "qconv2d_s8")
    return out


def qconv2d_s8_blockwise_f32(X: torch.Tensor, s_in: float, zp_in: int, blob: torch.Tensor,
                             info: PackedInfo, KH: int, KW: int, stride=(1, 1), pad=(0, 0, 0, 0),
                             dilation=(1, 1), bias=None, clamp_lo=-float("inf"),
                             clamp_hi=float("inf"), out=None):
    """Channel-blocked int8 convolution with f32 output (NHWC in and out)."""
    NB, H, W, Cc = X.shape
    OH = (H + pad[0] + pad[2] - (dilation[0] * (KH - 1) + 1)) // stride[0] + 1
    OW = (W + pad[1] + pad[3] - (dilation[1] * (KW - 1) + 1)) // stride[1] + 1
    x_desc = qtensor(QP_S8, [NB, H, W, Cc], scale=s_in, zero_point=zp_in)
    if out is None:
        out = torch.empty((NB, OH, OW, info.N), dtype=torch.float32, device=X.device)
    _check(_lib.qconv2d_s8_blockwise_f32(C.byref(x_desc), _ptr(X), C.byref(info), _ptr(blob), KH,
                                         KW, stride[0], stride[1], pad[0], pad[1], pad[2], pad[3],
                                         dilation[0], dilation[1], _ptr(bias), clamp_lo, clamp_hi,
                                         _ptr(out), _stream(X.device)),
           "qconv2d_s8_blockwise_f32")
    return out
