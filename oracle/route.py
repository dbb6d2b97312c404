"""Routing plan: expert offsets and the stable gather permutation.  ORACLE
(test infrastructure only).

The grouped GEMM runs every routing-dependent expert problem in one launch
(paper summary page, "3.4 Implementation details"); routed rows must
therefore be grouped by expert.  The plan is the plain stable counting sort
of the flat top-k ids (flat index i = t*k + j):

  counts[e]      = number of i with ids[i] == e
  offsets        = [0, cumsum(counts)]                  (E+1 entries)
  perm[r]        = i, the r-th flat index in (expert, i) order
  inv_perm[i]    = r  with perm[r] == i
"""
from __future__ import annotations

import numpy as np


def route(topk_ids: np.ndarray, E: int):
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    if ((ids < 0) | (ids >= E)).any():
        raise ValueError("expert id out of range")
    counts = np.bincount(ids, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(ids, kind="stable").astype(np.int32)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(len(perm), dtype=np.int32)
    return offsets, perm, inv_perm
