"""Value codes: E2M1 (FP4), E4M3 (FP8) and bf16 rounding.  ORACLE (test
infrastructure only).

The pages only name the formats (kept values on the FP4 E2M1 grid, one
unsigned E4M3 scale per 32 logical weights: paper summary page, "A
Sparse-quantized representation", Blackwell paired 4:8 NVFP4 / Storage
layout) and cite the OCP Microscaling formats paper for them.  The definitions used here are the
standard ones of those formats:

  E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
        exponent field 0 is subnormal: 0.5 * m.
  E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; the all-ones
        exponent with mantissa 7 is NaN (no inf); field 0 is subnormal:
        2^-6 * m/8.
"""
from __future__ import annotations

import numpy as np


def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e4m3_decode(code: int) -> float:
    """Value of an 8-bit E4M3 code (sign bit 7, exponent bits 6..3, mantissa 2..0)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


E2M1_VALUES = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)
E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)

# non-negative finite E4M3 codes 0x00..0x7E in ascending value order
_E4M3_POS = E4M3_VALUES[:0x7F]
E4M3_MAX = float(_E4M3_POS[-1])            # 448
_E2M1_POS = E2M1_VALUES[:8]                # 0, .5, 1, 1.5, 2, 3, 4, 6
E2M1_MAX = float(_E2M1_POS[-1])            # 6


def _nearest_even(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to x (x >= 0, grid ascending, codes =
    indices); on a tie the even index wins (round half to even mantissa).
    Values above the last grid point saturate to it."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (x < 0).any():
        raise ValueError("expects finite non-negative inputs")
    top = len(grid) - 1
    i = np.clip(np.searchsorted(grid, x, side="right") - 1, 0, top)
    j = np.minimum(i + 1, top)
    d_lo = x - grid[i]            # exact: x is fp32, grid values are short dyadics
    d_hi = grid[j] - x
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 1))
    out = np.where(pick_hi & (j != i), j, i)
    out = np.where(x >= grid[top], top, out)
    return out.astype(np.uint8)


def e4m3_encode(x) -> np.ndarray:
    """Round non-negative fp32 values to E4M3 codes: nearest, ties to even,
    saturating at 448 (never NaN)."""
    return _nearest_even(x, _E4M3_POS)


def e2m1_encode(x) -> np.ndarray:
    """Round fp32 values to E2M1 codes: nearest magnitude, ties to even,
    saturating at 6; a result of magnitude 0 is +0 (code 0)."""
    x = np.asarray(x, dtype=np.float64)
    mag = _nearest_even(np.abs(x), _E2M1_POS)
    neg = (x < 0) & (mag != 0)
    return (mag | (neg.astype(np.uint8) << 3)).astype(np.uint8)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits,
    exponent range of fp32), ties to even, overflow to +-inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| = m * 2^e, m in [0.5, 1)
    q = np.maximum(e - 8, -133)              # quantum of the bf16 neighbourhood
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
