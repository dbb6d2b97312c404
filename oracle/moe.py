"""Dispatch, grouped expert GEMM, SwiGLU and combine in float64.  ORACLE (test
infrastructure only).

Paper summary page:
  * "3.4 Implementation details": grouped GEMM over all routed expert
    problems in one launch, expert weights as the sparse operand.
  * "D.1 Implementation details": dispatch feeds the first expert GEMM,
    SwiGLU output preparation feeds the second, then scatter/combine.
  * "D.3 End-to-end serving benchmark": how tokens are combined and how the
    output is laid out is decided outside the expert kernel and kept the
    same for every backend.

Y[r, :] = X_routed[r, :] @ W_e^T for the expert e owning routed row r; the
inputs are the bf16 tokens (exact in float64) and the exactly decoded expert
matrices, so the only rounding here is float64 summation.
"""
from __future__ import annotations

from typing import Callable

import numpy as np

from .formats import bf16_round


def permute(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """Dispatch: X_routed[r] = X[perm[r] // k]."""
    return np.asarray(x)[np.asarray(perm) // k]


def expert_gemm(x_rows: np.ndarray, W: np.ndarray) -> np.ndarray:
    """x_rows [m, K] times W^T with W [N, K], float64."""
    return np.asarray(x_rows, np.float64) @ np.asarray(W, np.float64).T


def grouped_gemm(x_routed: np.ndarray, offsets: np.ndarray,
                 weight_of: Callable[[int], np.ndarray]) -> np.ndarray:
    """Y[off_e:off_e+M_e] = X_routed[off_e:off_e+M_e] @ W_e^T for every expert
    with rows; weight_of(e) returns the dense float64 W_e [N, K]."""
    E = len(offsets) - 1
    M = int(offsets[-1])
    Y = None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b <= a:
            continue
        W = weight_of(e)
        if Y is None:
            Y = np.zeros((M, W.shape[0]), np.float64)
        Y[a:b] = expert_gemm(x_routed[a:b], W)
    return Y


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x)), float64."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(y1: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up with gate = columns [0, N/2), up = [N/2, N)."""
    n2 = y1.shape[1] // 2
    return silu(y1[:, :n2]) * y1[:, n2:]


def unpermute(y: np.ndarray, inv_perm: np.ndarray, weights, T: int, k: int) -> np.ndarray:
    """Combine.  weights None: the routed rows back in flat order,
    out[i] = Y[inv_perm[i]] for i = t*k + j.  Otherwise
    out[t] = sum_{j<k} w[t*k+j] * Y[inv_perm[t*k+j]], summed in j order."""
    y = np.asarray(y, np.float64)
    inv = np.asarray(inv_perm)
    if weights is None:
        return y[inv]
    w = np.asarray(weights, np.float64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[inv.reshape(T, k)[:, j]]
    return out


def moe_chain(x: np.ndarray, offsets, perm, inv_perm, k: int,
              w_up: Callable[[int], np.ndarray], w_down: Callable[[int], np.ndarray],
              topk_weights=None):
    """permute -> gate/up GEMM -> SwiGLU (stored as bf16) -> down GEMM ->
    combine.  Returns (Y1, h, Y2, out) in float64; h is bf16-rounded because
    the hidden activation crosses the interface as a bf16 tensor."""
    T = x.shape[0]
    xr = permute(np.asarray(x, np.float64), perm, k)
    y1 = grouped_gemm(xr, offsets, w_up)
    h = bf16_round(swiglu(y1))
    y2 = grouped_gemm(h, offsets, w_down)
    out = unpermute(y2, inv_perm, topk_weights, T, k)
    return y1, h, y2, out
