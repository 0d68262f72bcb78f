"""fp64 CPU oracle of the deterministic GEMM: forward, input gradient and
weight gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: RL-Kernel PR #395, "feat(musa): add native deterministic gemm
kernel", summary and its list of changes: the forward is [M, K] @ [N, K]^T
without materialising the transposed right-hand side; dA = dC . B (the
input gradient, [M, K]); the weight gradient in the forward's [N, K] layout
(dB = dC^T . A); the reduction runs over the contraction index in a fixed
ascending order with fp32 accumulation, and the accuracy reference of the
page is an fp32 matmul followed by a bf16 conversion.

The oracle is the plain definition of each product in float64 from the exact
values of the bf16 inputs (a bf16 x bf16 product is exact in float64, and a
float64 sum of at most 2^20 of them is within a few units of 2^-53 of the
exact value).  ``abs_product`` gives the matching sums of |products|, which
bound the rounding error of any fp32 accumulation of the same terms.
"""

from __future__ import annotations

import math
from typing import Tuple

import numpy as np

from .linear_logp import to_f64

__all__ = ["det_gemm_fwd", "det_gemm_da", "det_gemm_db", "abs_product", "brute_force_fwd"]


def _mat(x) -> np.ndarray:
    m = to_f64(x)
    if m is None or m.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return m


def det_gemm_fwd(a, b) -> np.ndarray:
    """C[M, N] = A[M, K] . B[N, K]^T in float64 (reduction over K)."""
    A, B = _mat(a), _mat(b)
    if A.shape[1] != B.shape[1]:
        raise ValueError("A and B must share K")
    return A @ B.T


def det_gemm_da(dc, b) -> np.ndarray:
    """dA[M, K] = dC[M, N] . B[N, K] in float64 (reduction over N)."""
    G, B = _mat(dc), _mat(b)
    if G.shape[1] != B.shape[0]:
        raise ValueError("dC and B must share N")
    return G @ B


def det_gemm_db(a, dc) -> np.ndarray:
    """dB[N, K] = dC[M, N]^T . A[M, K] in float64 (reduction over M)."""
    A, G = _mat(a), _mat(dc)
    if A.shape[0] != G.shape[0]:
        raise ValueError("A and dC must share M")
    return G.T @ A


def abs_product(which: str, x, y) -> np.ndarray:
    """Sum of |terms| for each output of ``which`` in {"fwd", "da", "db"} with
    the same operands as the matching function: the scale of the rounding
    error of an fp32 accumulation."""
    X, Y = np.abs(_mat(x)), np.abs(_mat(y))
    if which == "fwd":
        return X @ Y.T
    if which == "da":
        return X @ Y
    if which == "db":
        return Y.T @ X
    raise ValueError(which)


def brute_force_fwd(a, b) -> Tuple[list, ...]:
    """C = A . B^T with plain Python floats and ``math.fsum`` (tiny inputs)."""
    A, B = _mat(a), _mat(b)
    M, K = A.shape
    N = B.shape[0]
    return [[math.fsum(float(A[m, k]) * float(B[n, k]) for k in range(K)) for n in range(N)]
            for m in range(M)]
