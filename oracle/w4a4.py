"""NVFP4 activation quantization and the W4A4 expert GEMM.  ORACLE (test
infrastructure only).

Paper summary page:
  * "D.1 Implementation details": the serving integration fuses dispatch with
    activation quantization for the first expert GEMM; the sparse backend's
    activation quantization forms 32-element scale blocks.
  * "3.4 Implementation details": the kernel packs weights and quantized
    activations in corresponding scale blocks.
  * "B Experimental setup", Compression scope: the target is paired 4:8
    NVFP4 W4A4 with 32-element scale blocks.

So an activation row x[t, :] (K % 32 == 0) is stored as E2M1 codes with one
E4M3 scale per 32 consecutive K positions -- the same K blocks as the weight
scales.  The pages name no second-level scale for activations; the reading
here (as for the weights, two levels, but per token row so that a row is
quantized on its own, in one pass, as a fused dispatch needs) is one fp32
scale per row.  Every decision is taken in fp32, in this order:
  g_t   = amax_t / 2688              (amax over the row; g_t = 1 if amax_t == 0)
  six_g = 6 * g_t
  s_b   = E4M3(amax_b / six_g)       per 32-position block (ties to even, 448 max)
  q     = E2M1(x / (value(s_b) * g_t)), 0 when value(s_b) * g_t == 0
and the activation the GEMM sees is  x~ = E2M1(q) * E4M3(s_b) * g_t  (exact in
float64).  The W4A4 GEMM is the float64 product of these dequantized rows
with the dequantized expert weights: the only rounding is the summation.

Byte layout of a quantized row block [T, K]:
  codes  [T, K/2]   two E2M1 codes per byte, position 2i in the low nibble
  scales [T, K/32]  E4M3 codes (sign 0)
  g      [T]        fp32
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import E2M1_VALUES, E4M3_VALUES, e2m1_encode, e4m3_encode


@dataclasses.dataclass
class PackedActivations:
    codes: np.ndarray    # uint8 [T, K/2]
    scales: np.ndarray   # uint8 [T, K/32]
    g: np.ndarray        # float32 [T]

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes + self.g.nbytes


def quantize_activations(x) -> PackedActivations:
    """NVFP4 quantization of activation rows x [T, K] (finite values, taken
    as fp32; bf16 inputs are exact), one row at a time."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    T, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    a = np.abs(x)
    amax = a.max(axis=1) if K else np.zeros(T, np.float32)
    g = np.where(amax > 0, (amax / np.float32(2688.0)).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    six_g = (np.float32(6.0) * g).astype(np.float32)
    amax_blk = a.reshape(T, K // 32, 32).max(axis=2)
    s_code = e4m3_encode((amax_blk / six_g[:, None]).astype(np.float32))
    sg = (E4M3_VALUES[s_code].astype(np.float32) * g[:, None]).astype(np.float32)
    sg_full = np.repeat(sg, 32, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sg_full > 0, x / np.where(sg_full > 0, sg_full, 1), 0).astype(np.float32)
    c = e2m1_encode(q)
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return PackedActivations(codes, s_code.astype(np.uint8), g)


def decode_activations(p: PackedActivations, include_row_scale: bool = True) -> np.ndarray:
    """x~[t, k] = E2M1(code) * E4M3(scale of k's block) (* g_t), float64."""
    T, K2 = p.codes.shape
    c = np.empty((T, 2 * K2), np.uint8)
    c[:, 0::2] = p.codes & 15
    c[:, 1::2] = p.codes >> 4
    v = E2M1_VALUES[c] * np.repeat(E4M3_VALUES[p.scales], 32, axis=1)
    if include_row_scale:
        v = v * p.g.astype(np.float64)[:, None]
    return v


def w4a4_expert_gemm(x_rows, W: np.ndarray) -> np.ndarray:
    """Rows of activations x_rows [m, K] quantized to NVFP4 and dequantized,
    times W^T with W [N, K] (the dequantized expert weights), float64."""
    xq = decode_activations(quantize_activations(x_rows))
    return xq @ np.asarray(W, np.float64).T
