"""Scatter fused into the GEMM epilogue (MOESQ_OUT_FLAT): the gather GEMM
and the fused routing + GEMM with rows stored at y[perm[r]] give exactly
the routed-order result reordered to flat order by the oracle's combine
without weights (float64 on the host), for 4:8 and paired weights, plain and
SwiGLU epilogues, at the workload shapes and on a batch with invalid routing
entries."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import f64, pack_workload


def _flat_ref(y_routed, ids, E, T, k):
    """The routed rows in flat order t*k + j, by the oracle's routing plan and
    combine."""
    _, _, inv_r = oracle.route(ids, E)
    return oracle.unpermute(f64(y_routed), inv_r, None, T, k)


@pytest.mark.gpu
@pytest.mark.parametrize("name,swiglu,paired", [
    ("tiny", False, False), ("decode-30b", False, False), ("decode-30b", False, True),
    ("prefill-30b", False, False), ("prefill-30b", False, True),
    ("decode-1t", True, False), ("decode-1t", True, True),
])
def test_gather_flat_matches_unpermute(lib, name, swiglu, paired):
    wl = synth.WORKLOADS[name]
    print(f"[{name}] gather GEMM, flat output, paired={paired}", flush=True)
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    x = synth.tokens(wl).cuda()
    epi = lib.EPI_SWIGLU if swiglu else lib.EPI_NONE
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    y = lib.grouped_spgemm_gather(x, perm, wl.k, off, w, epi)
    ref = _flat_ref(y, ids, wl.E, wl.T, wl.k)
    flat = torch.full_like(y, 7)   # every row must be overwritten
    lib.grouped_spgemm_gather(x, perm, wl.k, off, w, epi | lib.OUT_FLAT, out=flat)
    torch.cuda.synchronize()
    assert np.array_equal(f64(flat), ref), name


@pytest.mark.gpu
@pytest.mark.parametrize("name,swiglu,paired", [
    ("decode-30b", False, False), ("decode-30b", False, True), ("decode-1t", True, False),
    ("tiny", False, False),   # tiny: not a decode batch, the call's two-step fallback
])
def test_fused_route_flat_matches_unpermute(lib, name, swiglu, paired):
    wl = synth.WORKLOADS[name]
    print(f"[{name}] fused routing + GEMM, flat output, paired={paired}", flush=True)
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    x = synth.tokens(wl).cuda()
    epi = lib.EPI_SWIGLU if swiglu else lib.EPI_NONE
    ids_d = torch.from_numpy(ids).cuda()
    y, off, perm, inv = lib.route_grouped_spgemm(ids_d, x, wl.k, w, epi)
    ref = _flat_ref(y, ids, wl.E, wl.T, wl.k)
    flat = torch.full_like(y, 7)
    _, off2, perm2, inv2 = lib.route_grouped_spgemm(ids_d, x, wl.k, w, epi | lib.OUT_FLAT,
                                                    out=flat)
    torch.cuda.synchronize()
    assert torch.equal(off2, off) and torch.equal(perm2, perm) and torch.equal(inv2, inv)
    assert np.array_equal(f64(flat), ref), name


@pytest.mark.gpu
def test_flat_with_invalid_routing_entries(lib):
    """Routed rows whose perm entry is out of range have no flat destination:
    nothing is stored for them, every other flat row is the unpermuted one."""
    wl = synth.WORKLOADS["decode-30b"]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0))
    x = synth.tokens(wl).cuda()
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    y = lib.grouped_spgemm_gather(x, perm, wl.k, off, w, lib.EPI_NONE)
    ref = torch.from_numpy(_flat_ref(y, ids, wl.E, wl.T, wl.k)).cuda()
    bad = perm.clone()
    lost = [3, 40, wl.M - 1]                      # routed rows given invalid entries
    gone = perm[lost].long()                      # their flat rows, now written by nobody
    bad[lost] = torch.tensor([-1, wl.M, 1 << 20], dtype=torch.int32, device=bad.device)
    flat = torch.full_like(y, 7)
    lib.grouped_spgemm_gather(x, bad, wl.k, off, w, lib.EPI_NONE | lib.OUT_FLAT, out=flat)
    torch.cuda.synchronize()
    keep = torch.ones(wl.M, dtype=torch.bool, device=flat.device)
    keep[gone] = False
    assert torch.equal(flat[keep].double(), ref[keep])
    assert bool((flat[~keep] == 7).all())
