"""Integer affine GEMM through an fp64 library matmul -- a second formulation
of the oracle's O1 for full-size checks, where the scalar C loops would take
minutes.

TEST INFRASTRUCTURE (same rules as ``oracle.c``).  Definition followed: the
integer affine product of "Quantized GEMM: numeric contract, SRAM, DMA and
result verification" section 1, acc = sum_k (A-zA)(B-zB) + bias.  Every
operand is an integer of magnitude <= 255, so each product is <= 65025 and
any sum over K < 2^53 / 65025 terms is exact in fp64; the matmul therefore
returns the integer result exactly, whatever its summation order.
"""
from __future__ import annotations

import numpy as np

_EXACT_K_LIMIT = (1 << 53) // 65025


def gemm_affine_f64(A, zA, B_nk, zB, bias=None, rows=None):
    """acc[M,N] int64 = (A - zA) @ (B_nk - zB[:,None]).T + bias, exactly.

    ``B_nk`` is [N, K]; ``rows`` optionally restricts to a subset of A's rows."""
    A = np.asarray(A)
    if rows is not None:
        A = A[rows]
    K = A.shape[1]
    assert K < _EXACT_K_LIMIT
    Af = A.astype(np.float64) - float(zA)
    zb = np.broadcast_to(np.asarray(zB, dtype=np.float64), (B_nk.shape[0],))
    Bf = np.asarray(B_nk).astype(np.float64) - zb[:, None]
    acc = Af @ Bf.T
    if bias is not None:
        acc += np.asarray(bias, dtype=np.float64)[None, :]
    return acc.astype(np.int64)
