"""Seeded synthetic inputs for the grouped 4:8 FP4 expert GEMM.

This module only draws inputs: dense expert weights, tokens, router logits
and the top-k routing that a MoE router would produce.  It holds none of the
compressed-format arithmetic (no quantisation, no decode, no GEMM); both the
HIP library and the CPU oracle take what it returns and do their own work.

The workloads mirror the expert shapes of the pages' kernel benchmark
(Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE,
"D.2 Kernel benchmark": 30B-class and trillion-class gate/up and down
projections) at the sizes given in the workload table below.  There are no
trained weights or routers here; every tensor is synthetic.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "child_seed", "tokens", "routing",
           "dense_expert", "dense_experts"]

WEIGHT_STD = 0.02          # dense expert weights ~ N(0, 0.02^2)
OUTLIER_FRACTION = 0.01    # 1 % of activation channels ...
OUTLIER_GAIN = 10.0        # ... scaled by 10 before the bf16 cast
ZIPF_S = 1.1               # expert-load exponent of the prefill workloads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int                      # experts
    T: int                      # tokens
    k: int                      # experts per token
    proj: tuple                 # ((name, N, K), ...) in execution order
    outliers: bool              # 1 % outlier channels in the activations
    bias: str                   # "none" | "gauss" | "zipf"
    seed: int
    swiglu: bool = False        # gate+up -> SwiGLU -> down chain
    weighted_combine: bool = False

    @property
    def M(self) -> int:
        return self.T * self.k

    @property
    def K_in(self) -> int:
        return self.proj[0][2]


WORKLOADS = {
    "tiny": Workload("tiny", E=8, T=64, k=2, proj=(("w", 128, 256),),
                     outliers=False, bias="none", seed=1000),
    "decode-30b": Workload("decode-30b", E=128, T=16, k=8,
                           proj=(("gate_up", 1536, 2048),),
                           outliers=True, bias="gauss", seed=1001),
    "prefill-30b": Workload("prefill-30b", E=128, T=4096, k=8,
                            proj=(("gate_up", 1536, 2048),),
                            outliers=True, bias="zipf", seed=1002),
    "decode-1t": Workload("decode-1t", E=384, T=64, k=8,
                          proj=(("gate_up", 4096, 7168), ("down", 7168, 2048)),
                          outliers=True, bias="gauss", seed=1003, swiglu=True),
    "prefill-1t": Workload("prefill-1t", E=384, T=8192, k=8,
                           proj=(("gate_up", 4096, 7168), ("down", 7168, 2048)),
                           outliers=True, bias="zipf", seed=1004, swiglu=True,
                           weighted_combine=True),
}


def child_seed(seed: int, *tags: int) -> int:
    """A 63-bit seed derived from (seed, *tags) with numpy's SeedSequence."""
    st = np.random.SeedSequence([int(seed)] + [int(t) for t in tags])
    a, b = st.generate_state(2, dtype=np.uint32)
    return ((int(a) << 32) | int(b)) & ((1 << 63) - 1)


# tags for child seeds
_TAG_TOKENS, _TAG_OUTLIER, _TAG_LOGITS, _TAG_BIAS, _TAG_RANK, _TAG_W = 1, 2, 3, 4, 5, 6


def tokens(wl: Workload, T: int | None = None, K: int | None = None,
           seed: int | None = None) -> torch.Tensor:
    """bf16 [T, K] activations: N(0,1) in fp32, outlier channels x10, then the
    round-to-nearest-even bf16 cast.  Returned on the CPU."""
    T = wl.T if T is None else T
    K = wl.K_in if K is None else K
    seed = wl.seed if seed is None else seed
    g = torch.Generator().manual_seed(child_seed(seed, _TAG_TOKENS))
    x = torch.randn(T, K, generator=g, dtype=torch.float32)
    if wl.outliers:
        n_out = int(round(OUTLIER_FRACTION * K))
        rng = np.random.default_rng(child_seed(seed, _TAG_OUTLIER))
        ch = np.sort(rng.choice(K, size=n_out, replace=False))
        x[:, torch.from_numpy(ch)] *= OUTLIER_GAIN
    return x.to(torch.bfloat16)


def _topk_stable(score: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row; equal scores -> lower index."""
    return np.argsort(-score, axis=1, kind="stable")[:, :k]


def _loads(ids: np.ndarray, E: int) -> np.ndarray:
    return np.bincount(ids.reshape(-1), minlength=E)


def _zipf_slope(loads: np.ndarray) -> float:
    nz = np.sort(loads[loads > 0])[::-1].astype(np.float64)
    hi = max(3, len(nz) // 2)
    r = np.arange(1, len(nz) + 1, dtype=np.float64)[1:hi]
    y = nz[1:hi]
    A = np.stack([np.log(r), np.ones_like(r)], axis=1)
    return float(np.linalg.lstsq(A, np.log(y), rcond=None)[0][0])


def _zipf_bias(logits: np.ndarray, E: int, k: int, seed: int) -> np.ndarray:
    """Per-expert router bias b_e = -s*c*ln(rank_e), with the bottom E//25
    ranks forced to zero load, c found by bisection so that the log-log slope
    of the realised loads is -s."""
    rng = np.random.default_rng(child_seed(seed, _TAG_RANK))
    rank = rng.permutation(E) + 1
    dead = rank > E - E // 25

    def bias_for(c: float) -> np.ndarray:
        b = (-ZIPF_S * c * np.log(rank.astype(np.float64))).astype(np.float32)
        b[dead] = np.float32(-1e9)
        return b

    def fast_loads(c: float) -> np.ndarray:
        # the tie order of top-k does not move the loads of random logits
        sc = logits + bias_for(c)
        return _loads(np.argpartition(-sc, k - 1, axis=1)[:, :k], E)

    lo, hi = 0.0, 4.0
    for _ in range(30):
        c = 0.5 * (lo + hi)
        sl = _zipf_slope(fast_loads(c))
        if sl > -ZIPF_S:
            lo = c
        else:
            hi = c
    return bias_for(0.5 * (lo + hi))


def routing(wl: Workload, T: int | None = None, seed: int | None = None):
    """Top-k routing as a MoE router produces it.

    Returns (topk_ids int32 [T*k], topk_weights fp32 [T*k]) in flat token-major
    order i = t*k + j.  Weights are the softmax of the selected scores,
    renormalised over the k chosen experts (computed in float64)."""
    T = wl.T if T is None else T
    seed = wl.seed if seed is None else seed
    E, k = wl.E, wl.k
    rng = np.random.default_rng(child_seed(seed, _TAG_LOGITS))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.bias == "none":
        bias = np.zeros(E, np.float32)
    elif wl.bias == "gauss":
        bias = np.random.default_rng(child_seed(seed, _TAG_BIAS)).standard_normal(
            E, dtype=np.float32)
    elif wl.bias == "zipf":
        bias = _zipf_bias(logits, E, k, seed)
    else:
        raise ValueError(wl.bias)
    score = logits + bias
    ids = _topk_stable(score, k)
    sel = np.take_along_axis(score, ids, axis=1).astype(np.float64)
    sel -= sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w /= w.sum(axis=1, keepdims=True)
    return (np.ascontiguousarray(ids.reshape(-1), dtype=np.int32),
            np.ascontiguousarray(w.reshape(-1), dtype=np.float32))


def load_stats(ids: np.ndarray, E: int) -> dict:
    loads = _loads(ids, E)
    return {"active": int((loads > 0).sum()), "zero": int((loads == 0).sum()),
            "max": int(loads.max()), "over_1000": int((loads > 1000).sum()),
            "slope": _zipf_slope(loads) if (loads > 0).sum() > 4 else float("nan")}


def dense_expert(wl: Workload, proj: int, e: int, device="cpu",
                 N: int | None = None, K: int | None = None,
                 seed: int | None = None) -> torch.Tensor:
    """Dense fp32 [N, K] weights of expert e of projection `proj`, N(0, 0.02^2).

    Each (projection, expert) has its own generator, so any expert can be
    regenerated alone.  The values depend on `device` (torch's CPU and GPU
    generators differ); callers hand the same tensor to both sides."""
    _, N0, K0 = wl.proj[proj]
    N = N0 if N is None else N
    K = K0 if K is None else K
    seed = wl.seed if seed is None else seed
    g = torch.Generator(device=device).manual_seed(child_seed(seed, _TAG_W, proj, e))
    w = torch.randn(N, K, generator=g, dtype=torch.float32, device=device)
    return w.mul_(WEIGHT_STD)


def dense_experts(wl: Workload, proj: int, experts=None, device="cpu", **kw):
    experts = range(wl.E) if experts is None else experts
    return torch.stack([dense_expert(wl, proj, e, device=device, **kw) for e in experts])
