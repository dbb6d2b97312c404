"""Helpers of the GPU parity tests: tolerance check, building a workload's
inputs on the GPU, and oracle references for sampled experts."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

# Tolerance of the bf16 outputs against the float64 oracle, per tensor:
# relative Frobenius error and max abs error relative to max |ref|.
REL_FRO = 5e-3
MAX_ABS_REL = 1e-2


def tol_check(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mx = np.abs(got - ref).max() if got.size else 0.0
    lim = MAX_ABS_REL * (np.abs(ref).max() if ref.size else 0.0)
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= lim, f"{what}: max abs error {mx:.3e} > {lim:.3e}"
    return rel, mx


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def pack_workload(m, wl, proj: int, chunk: int = 16, paired: bool = False):
    """Dense weights of every expert drawn on the GPU and packed there, a
    chunk of experts at a time (4:8, or paired 4:8).  Returns the library's
    canonical Weights."""
    _, N, K = wl.proj[proj]
    w = m.Weights.empty(wl.E, N, K, layout=m.LAYOUT_PAIRED if paired else m.LAYOUT_CANONICAL)
    pack = m.moesq_pack_weights_paired if paired else m.moesq_pack_weights
    for c0 in range(0, wl.E, chunk):
        c1 = min(wl.E, c0 + chunk)
        dense = synth.dense_experts(wl, proj, range(c0, c1), device="cuda")
        pack(dense, c1 - c0, N, K, w.values[c0:c1], w.masks[c0:c1], w.scales[c0:c1],
             w.global_scale[c0:c1])
        del dense
    return w


def oracle_expert(wl, proj: int, e: int, device="cuda", paired: bool = False):
    """The oracle's compression of the same dense weights (drawn on `device`
    exactly as pack_workload draws them, then moved to the CPU)."""
    dense = synth.dense_expert(wl, proj, e, device=device).cpu().numpy()
    return oracle.quantize_paired(dense) if paired else oracle.quantize(dense)


def oracle_decode(p, include_global=True):
    """Dense float64 matrix of an oracle-packed expert of either format."""
    if isinstance(p, oracle.PackedPairedExpert):
        return oracle.decode_paired(p, include_global)
    return oracle.decode(p, include_global)


def assert_same_pack(w, e: int, p, what=""):
    meta = p.patterns if isinstance(p, oracle.PackedPairedExpert) else p.masks
    assert np.array_equal(w.values[e].cpu().numpy(), p.values), f"{what}: values differ"
    assert np.array_equal(w.masks[e].cpu().numpy(), meta), f"{what}: masks/patterns differ"
    assert np.array_equal(w.scales[e].cpu().numpy(), p.scales), f"{what}: scales differ"
    assert w.global_scale[e].item() == float(p.g), f"{what}: global scale differs"


# Large grouped-GEMM calls split the experts over three launches by their own
# row counts: up to 16 rows, 17 to 32, and more.  Samples cover each range.
LAUNCH_RANGES = ((1, 16), (17, 32), (33, 1 << 30))


def pick_experts(counts, rng, n_random=1):
    """Experts to check: the largest, one from each launch range's row counts
    (the middle one of the range, in expert order), and a few random active
    ones."""
    active = np.nonzero(counts)[0]
    pick = {int(active[np.argmax(counts[active])])}
    for lo, hi in LAUNCH_RANGES:
        inr = active[(counts[active] >= lo) & (counts[active] <= hi)]
        if len(inr):
            pick.add(int(inr[len(inr) // 2]))
    for e in rng.choice(active, size=min(n_random, len(active)), replace=False):
        pick.add(int(e))
    return sorted(pick)


def oracle_experts(wl, proj: int, experts, paired: bool = False, threads: int = 16):
    """The oracle's compression and exact float64 decode of the given experts
    (dense weights drawn on the GPU exactly as pack_workload draws them), run
    on a pool of host threads.  Returns {e: (packed, decoded)}."""
    import concurrent.futures as cf
    dense = {int(e): synth.dense_expert(wl, proj, int(e), device="cuda").cpu().numpy()
             for e in experts}

    def one(e):
        p = oracle.quantize_paired(dense[e]) if paired else oracle.quantize(dense[e])
        return e, (p, oracle_decode(p))
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(one, list(dense)))
