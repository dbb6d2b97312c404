"""Compression of one dense expert matrix to the 4:8 / E2M1 / E4M3 format and
its exact decode.  ORACLE (test infrastructure only).

Follows the paper summary page, "3.4 Implementation details" (after the
scales are recomputed the packer stores the FP4 codes, the sparsity metadata
and one scale for each 32 logical weights) and "A Sparse-quantized representation" (each group of
eight keeps four values; 16 kept values of a 32-weight block share one scale;
zero lies on the grid so pruned positions are feasible).  The selection of
the support here is the hard top-4 by magnitude; the pages learn it, which is
offline work outside this path.

Byte layout of one expert W [N, K] (K % 32 == 0), row-major:
  values [N, K/4]  two E2M1 codes per byte, the group's four kept codes in
                   ascending position, the lower one in the low nibble
  masks  [N, K/8]  bit i set <=> position 8*g + i is kept (popcount 4)
  scales [N, K/32] E4M3 code of the block scale (sign 0)
  g      fp32      global scale of the expert matrix
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import E2M1_VALUES, E4M3_VALUES, e2m1_encode, e4m3_encode

E2M1_MAX = np.float32(6.0)
E4M3_MAX = np.float32(448.0)


@dataclasses.dataclass
class PackedExpert:
    values: np.ndarray   # uint8 [N, K/4]
    masks: np.ndarray    # uint8 [N, K/8]
    scales: np.ndarray   # uint8 [N, K/32]
    g: np.float32

    @property
    def nbytes(self) -> int:
        return self.values.nbytes + self.masks.nbytes + self.scales.nbytes + 4


def support(Wd: np.ndarray) -> np.ndarray:
    """Boolean keep-map [N, K]: in every group of 8 consecutive K positions
    the 4 largest |w|; equal magnitudes go to the lower position."""
    N, K = Wd.shape
    a = np.abs(Wd.astype(np.float32)).reshape(N, K // 8, 8)
    order = np.argsort(-a, axis=2, kind="stable")
    keep = np.zeros_like(a, dtype=bool)
    np.put_along_axis(keep, order[:, :, :4], True, axis=2)
    return keep.reshape(N, K)


def masks_of(keep: np.ndarray) -> np.ndarray:
    N, K = keep.shape
    bits = keep.reshape(N, K // 8, 8).astype(np.uint32) << np.arange(8, dtype=np.uint32)
    return bits.sum(axis=2).astype(np.uint8)


def quantize_kept(Wd: np.ndarray, keep: np.ndarray):
    """Codes of the kept weights of a dense fp32 [N, K] matrix under the
    keep-map `keep` [N, K] (four kept positions per group of 8).

    All arithmetic that decides a code is done in fp32, in this order:
      g     = amax / 2688          (2688 = 6 * 448; g = 1 if amax == 0)
      six_g = 6 * g
      s     = E4M3(amax_32 / six_g)             per 32-position block
      q     = E2M1(w / (value(s) * g))          per kept weight
    amax and amax_32 run over kept positions only.  Returns the kept codes
    [N, K/8, 4] (ascending position per group), the scale codes [N, K/32]
    and g."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    N, K = Wd.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    a = np.abs(Wd)
    amax = np.float32(a[keep].max()) if a.size else np.float32(0)
    g = np.float32(amax / np.float32(2688.0)) if amax > 0 else np.float32(1.0)
    six_g = np.float32(np.float32(6.0) * g)
    amax_blk = np.where(keep, a, np.float32(0)).reshape(N, K // 32, 32).max(axis=2)
    s_code = e4m3_encode((amax_blk / six_g).astype(np.float32))
    s_val = E4M3_VALUES[s_code].astype(np.float32)
    sg = (s_val * g).astype(np.float32)                      # [N, K/32]
    sg_full = np.repeat(sg, 32, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sg_full > 0, Wd / np.where(sg_full > 0, sg_full, 1), 0).astype(np.float32)
    codes = e2m1_encode(q)                                   # [N, K]
    kept = codes.reshape(N, K // 8, 8)[keep.reshape(N, K // 8, 8)].reshape(N, K // 8, 4)
    return kept.astype(np.uint8), s_code, g


def pack_nibbles(kept: np.ndarray) -> np.ndarray:
    """[N, K/8, 4] kept codes -> [N, K/4] bytes: kept values 0,1 in the first
    byte of the group, 2,3 in the second, the lower one in the low nibble."""
    N, G, _ = kept.shape
    values = np.empty((N, G, 2), np.uint8)
    values[:, :, 0] = kept[:, :, 0] | (kept[:, :, 1] << 4)
    values[:, :, 1] = kept[:, :, 2] | (kept[:, :, 3] << 4)
    return values.reshape(N, 2 * G)


def unpack_nibbles(values: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: [N, K/4] bytes -> [N, K/8, 4] codes."""
    N = values.shape[0]
    v = values.reshape(N, -1, 2)
    return np.stack([v[:, :, 0] & 15, v[:, :, 0] >> 4, v[:, :, 1] & 15, v[:, :, 1] >> 4], axis=2)


def quantize(Wd: np.ndarray) -> PackedExpert:
    """Compress a dense fp32 [N, K] expert matrix: the support of `support`,
    then the codes of `quantize_kept`."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    N, K = Wd.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    keep = support(Wd)
    kept, s_code, g = quantize_kept(Wd, keep)
    return PackedExpert(pack_nibbles(kept), masks_of(keep), s_code, g)


def decode_kept(codes4: np.ndarray, bits: np.ndarray, scales: np.ndarray, g,
                include_global: bool = True) -> np.ndarray:
    """Dense float64 [N, K] from the kept codes [N, K/8, 4] and the keep-map
    [N, K/8, 8] (four set per group): w = E2M1(c_j) * E4M3(s_b) (* g) at the
    j-th kept position of the group, 0 elsewhere.  Exact in float64."""
    N, G, _ = bits.shape
    K = 8 * G
    rank = np.clip(np.cumsum(bits, axis=2) - 1, 0, 3)          # index j of each kept position
    code = np.take_along_axis(codes4, rank, axis=2)
    val = np.where(bits, E2M1_VALUES[code], 0.0).reshape(N, K)
    w = val * np.repeat(E4M3_VALUES[scales], 32, axis=1)
    if include_global:
        w = w * np.float64(g)
    return w


def decode(p: PackedExpert, include_global: bool = True) -> np.ndarray:
    """Dense float64 [N, K] matrix the packed expert stands for:
    w[n, 8g+i] = E2M1(c_j) * E4M3(s_b) * g at the j-th set bit i of the mask,
    0 elsewhere.  Exact in float64."""
    bits = ((p.masks[:, :, None].astype(np.uint32) >> np.arange(8)) & 1).astype(bool)
    if (bits.sum(axis=2) != 4).any():
        raise ValueError("every mask byte must have exactly four bits set")
    return decode_kept(unpack_nibbles(p.values), bits, p.scales, p.g, include_global)
