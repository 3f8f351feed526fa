"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds only random-number generation and the input recipes (shapes,
value ranges, distributions).  It contains none of the quantized-matmul
arithmetic, and it imports neither the oracle nor the GPU library.

Generator: SplitMix64 in counter form -- output i of stream ``s`` is
``mix(s + (i+1)*0x9E3779B97F4A7C15)`` with Steele/Lea/Flood's published
finaliser -- so any slice of a stream can be produced independently.
  * integers in [lo, hi]: the top ceil(log2(range)) bits of each draw, with
    rejection of values >= range (no modulo bias);
  * f32 uniform in [lo, hi): ``(x >> 40) * 2^-24`` mapped affinely in fp64,
    then rounded to f32;
  * N(0,1): Box-Muller on two draws, in fp64, rounded to f32.
Each tensor of a workload draws from its own stream ``seed*1000 + tensor_id``.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def substream(seed: int, tensor_id: int) -> int:
    return (seed * 1000 + tensor_id) & 0xFFFFFFFFFFFFFFFF


def uniform_int(stream: int, shape, lo: int, hi: int, dtype=np.int32) -> np.ndarray:
    """Uniform integers in the closed range [lo, hi] by top-bits rejection."""
    n = int(np.prod(shape)) if len(tuple(np.atleast_1d(shape))) else 1
    rng = hi - lo + 1
    assert rng >= 1
    bits = max(1, math.ceil(math.log2(rng))) if rng > 1 else 1
    out = np.empty(n, dtype=np.int64)
    filled, pos = 0, 0
    while filled < n:
        want = n - filled
        chunk = want + want // 8 + 64 if (1 << bits) != rng else want
        x = splitmix64(stream, pos, chunk)
        pos += chunk
        v = (x >> np.uint64(64 - bits)).astype(np.int64)
        v = v[v < rng]
        take = min(v.shape[0], want)
        out[filled:filled + take] = v[:take] + lo
        filled += take
    return out.astype(dtype).reshape(shape)


def uniform_f32(stream: int, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    x = splitmix64(stream, 0, n)
    u = (x >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def normal_f32(stream: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    x = splitmix64(stream, 0, 2 * n)
    u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = (x[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return z.astype(np.float32).reshape(shape)


# --------------------------------------------------------------------------
# Workload recipes.  Shapes and distributions follow the five workloads the
# library is measured on; where a range is not given by them the reading used
# is noted (bias ranges, the large GEMM's activation scale).
# --------------------------------------------------------------------------
BASE_SEED = 0x51A7E0


def gemm_affine_per_tensor(seed=BASE_SEED + 0, M=130, N=70, K=129):
    """INT8 affine per-tensor GEMM: A [M,K], B [K,N] row-major, uniform int8,
    zA=3, zB=-5, sA=0.02, sB=0.01, s_out=0.5, zp_out=-2, bias U[-1000,1000]."""
    return dict(
        A=uniform_int(substream(seed, 1), (M, K), -128, 127, np.int8),
        B=uniform_int(substream(seed, 2), (K, N), -128, 127, np.int8),
        bias=uniform_int(substream(seed, 3), (N,), -1000, 1000, np.int32),
        zA=3, zB=-5, sA=0.02, sB=0.01, s_out=0.5, zp_out=-2, relu=False,
    )


def conv3x3_nhwc(seed=BASE_SEED + 1, H=56, W=56, C=64, OC=64, NB=1):
    """INT8 3x3 conv, stride 1, pad 1 (pad value = input zp): X NHWC uniform
    int8, zp_in=7, s_in=0.05; W OIHW uniform [-127,127]; per-channel weight
    scales U[0.001,0.01]; bias U[-1000,1000] (reading); ReLU; s_out=0.1,
    zp_out=0."""
    return dict(
        X=uniform_int(substream(seed, 1), (NB, H, W, C), -128, 127, np.int8),
        W=uniform_int(substream(seed, 2), (OC, C, 3, 3), -127, 127, np.int8),
        s_w=uniform_f32(substream(seed, 3), (OC,), 0.001, 0.01),
        bias=uniform_int(substream(seed, 4), (OC,), -1000, 1000, np.int32),
        zp_in=7, s_in=0.05, s_out=0.1, zp_out=0, relu=True,
        stride=(1, 1), pad=(1, 1, 1, 1),
    )


def a8w4(seed, M, N, K, group=32):
    """A8W4: X [M,K] N(0,1) f32; W [N,K] uniform int4 [-8,7]; group scales
    U[0.002,0.02]; bias U[-1,1] (reading); clamp [-6,6]."""
    return dict(
        X=normal_f32(substream(seed, 1), (M, K)),
        W=uniform_int(substream(seed, 2), (N, K), -8, 7, np.int8),
        sw=uniform_f32(substream(seed, 3), (N, (K + group - 1) // group), 0.002, 0.02),
        bias=uniform_f32(substream(seed, 4), (N,), -1.0, 1.0),
        clamp_lo=-6.0, clamp_hi=6.0, group=group,
    )


def a8w4_gemv(seed=BASE_SEED + 2):
    return a8w4(seed, 1, 4096, 4096)


def a8w4_gemm(M, seed=BASE_SEED + 3):
    return a8w4(seed, M, 11008, 4096)


def gemm_large(seed=BASE_SEED + 4, M=8192, N=8192, K=8192):
    """Large INT8 GEMM: A [M,K] uniform int8, zA=0, sA=0.01 (reading); W [N,K]
    symmetric uniform [-127,127] with per-channel scales U[0.001,0.01]; no bias
    (reading); int8 output scale 1.0, zp 0; also a raw int32 output."""
    return dict(
        A=uniform_int(substream(seed, 1), (M, K), -128, 127, np.int8),
        W=uniform_int(substream(seed, 2), (N, K), -127, 127, np.int8),
        s_w=uniform_f32(substream(seed, 3), (N,), 0.001, 0.01),
        zA=0, sA=0.01, s_out=1.0, zp_out=0, relu=False,
    )
