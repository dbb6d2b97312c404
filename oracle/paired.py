"""Compression of one dense expert matrix to the paired 4:8 / E2M1 / E4M3
format and its exact decode.  ORACLE (test infrastructure only).

Follows the paper summary page, "A Sparse-quantized representation":
  * Blackwell paired 4:8 NVFP4 -- of the four position pairs (2i, 2i+1) of
    a group of eight weights, two are kept, so six patterns are allowed;
    the 16 kept values of a 32-weight block share one UE4M3 scale and the
    kept values lie on the E2M1 grid.
  * Storage layout -- a group of eight stores its four kept codes and the
    number of its pattern, a 32-weight block one UE4M3 scale: 2.75 bits per
    weight.

Readings where the pages are silent:
  * pattern index: p in [0, 6) numbers the kept pair couples (i, j), i < j,
    in lexicographic order -- (0,1) (0,2) (0,3) (1,2) (1,3) (2,3);
  * selection: the two pairs with the largest |w_2i| + |w_2i+1| (the sum in
    fp32) are kept; equal sums go to the lower pair index (the pages learn
    the support offline; this is the plain magnitude rule, as for 4:8);
  * quantisation of the kept values: exactly as the 4:8 format (same global
    scale, block scales and E2M1 rounding, over kept positions only).

Byte layout of one expert W [N, K] (K % 32 == 0), row-major:
  values   [N, K/4]   four kept E2M1 codes per group in ascending position,
                      two per byte, the lower position in the low nibble
  patterns [N, K/16]  pattern index of group g in byte g/2, the even group in
                      the low nibble
  scales   [N, K/32]  E4M3 code of the block scale (sign 0)
  g        fp32       global scale of the expert matrix
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .pack import decode_kept, pack_nibbles, quantize_kept, unpack_nibbles

# kept pair couples, by pattern index
PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def pattern_mask(p: int) -> int:
    """8-bit keep-mask of pattern p (bit i <-> position i of the group)."""
    i, j = PAIRS[p]
    return (3 << (2 * i)) | (3 << (2 * j))


@dataclasses.dataclass
class PackedPairedExpert:
    values: np.ndarray    # uint8 [N, K/4]
    patterns: np.ndarray  # uint8 [N, K/16]
    scales: np.ndarray    # uint8 [N, K/32]
    g: np.float32

    @property
    def nbytes(self) -> int:
        return self.values.nbytes + self.patterns.nbytes + self.scales.nbytes + 4


def paired_pattern(Wd: np.ndarray) -> np.ndarray:
    """Pattern index [N, K/8] of every group: the two pairs with the largest
    fp32 |w| sums; equal sums go to the lower pair index."""
    N, K = Wd.shape
    a = np.abs(np.asarray(Wd, np.float32)).reshape(N, K // 8, 4, 2)
    pair = (a[..., 0] + a[..., 1]).astype(np.float32)        # [N, K/8, 4], fp32 sums
    order = np.argsort(-pair, axis=2, kind="stable")          # stable: lower index first on ties
    i = np.minimum(order[..., 0], order[..., 1])
    j = np.maximum(order[..., 0], order[..., 1])
    lookup = np.full((4, 4), 255, np.uint8)
    for p, (pi, pj) in enumerate(PAIRS):
        lookup[pi, pj] = p
    return lookup[i, j]


def paired_support(Wd: np.ndarray) -> np.ndarray:
    """Boolean keep-map [N, K] of the paired patterns."""
    pat = paired_pattern(Wd)
    masks = np.array([pattern_mask(p) for p in range(6)], np.uint32)[pat]
    N, G = pat.shape
    return (((masks[:, :, None] >> np.arange(8)) & 1).astype(bool)).reshape(N, 8 * G)


def quantize_paired(Wd: np.ndarray) -> PackedPairedExpert:
    """Compress a dense fp32 [N, K] expert matrix to the paired format."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    N, K = Wd.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    pat = paired_pattern(Wd)
    keep = paired_support(Wd)
    kept, s_code, g = quantize_kept(Wd, keep)
    pp = pat.reshape(N, K // 16, 2)
    patterns = (pp[:, :, 0] | (pp[:, :, 1] << 4)).astype(np.uint8)
    return PackedPairedExpert(pack_nibbles(kept), patterns, s_code, g)


def decode_paired(p: PackedPairedExpert, include_global: bool = True) -> np.ndarray:
    """Dense float64 [N, K]: w[n, 8g+i] = E2M1(c_j) * E4M3(s_b) * g at the
    j-th kept position i of pattern p_g, 0 elsewhere.  Exact in float64."""
    N = p.patterns.shape[0]
    pat = np.stack([p.patterns & 15, p.patterns >> 4], axis=2).reshape(N, -1)   # [N, K/8]
    if (pat > 5).any():
        raise ValueError("pattern indices must lie in [0, 6)")
    masks = np.array([pattern_mask(q) for q in range(6)], np.uint32)[pat]
    bits = ((masks[:, :, None] >> np.arange(8)) & 1).astype(bool)
    return decode_kept(unpack_nibbles(p.values), bits, p.scales, p.g, include_global)
