"""moesq_route_grouped_spgemm: routing + dispatch + grouped GEMM of a decode
batch in one launch gives exactly moesq_route followed by
moesq_grouped_spgemm_gather (plan and output bytes), for 4:8 and paired
weights, with invalid ids, on the fallback path (batches too large to route
inside the GEMM) and for an empty batch; one case against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import f64, oracle_decode, oracle_expert, pack_workload, tol_check


def _two_step(lib, ids_d, x, k, w, epi):
    off, perm, inv = lib.route(ids_d, w.E, k)
    y = lib.grouped_spgemm_gather(x, perm, k, off, w, epi)
    return y, off, perm, inv


def _same(lib, ids_d, x, k, w, epi, what):
    y1, off1, perm1, inv1 = lib.route_grouped_spgemm(ids_d, x, k, w, epi)
    y2, off2, perm2, inv2 = _two_step(lib, ids_d, x, k, w, epi)
    torch.cuda.synchronize()
    assert torch.equal(off1, off2), what
    rows = int(off2[-1].item())
    assert torch.equal(perm1[:rows], perm2[:rows]), what
    assert torch.equal(inv1, inv2), what
    assert torch.equal(y1[:rows], y2[:rows]), what     # rows past the experts are not written


@pytest.mark.gpu
@pytest.mark.parametrize("name,swiglu,paired", [
    ("decode-30b", False, False), ("decode-30b", False, True),
    ("decode-1t", True, False), ("decode-1t", True, True),
])
def test_fused_matches_two_calls(lib, name, swiglu, paired):
    wl = synth.WORKLOADS[name]
    print(f"[{name}] fused route + GEMM, paired={paired}", flush=True)
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    x = synth.tokens(wl).cuda()
    epi = lib.EPI_SWIGLU if swiglu else lib.EPI_NONE
    ids_d = torch.from_numpy(ids).cuda()
    _same(lib, ids_d, x, wl.k, w, epi, name)
    # invalid ids are dropped from the plan, as moesq_route drops them
    bad = ids_d.clone()
    bad[[0, 5, wl.M - 1]] = torch.tensor([-1, wl.E, 1 << 20], dtype=torch.int32, device=bad.device)
    _same(lib, bad, x, wl.k, w, epi, name + " with invalid ids")


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 13, 125, 128])
def test_fused_row_counts(lib, T):
    # routed-row counts from one id to the fused maximum (T*k = 1024), ragged
    # against the 64 ids of a wave
    wl = synth.WORKLOADS["decode-1t"]
    print(f"[decode-1t T={T}] fused route + GEMM, M={T * wl.k}", flush=True)
    ids, _ = synth.routing(wl, T=T, seed=wl.seed + T)
    w = lib.tile_weights(pack_workload(lib, wl, 1))
    x = synth.tokens(wl, T=T, K=wl.proj[1][2], seed=wl.seed + T).cuda()
    _same(lib, torch.from_numpy(ids).cuda(), x, wl.k, w, lib.EPI_NONE, f"T={T}")


@pytest.mark.gpu
@pytest.mark.parametrize("E,T,k,flat", [(1, 3, 1, False), (7, 4, 7, True), (1000, 128, 8, False),
                                        (1024, 100, 8, True)])
def test_fused_expert_counts(lib, E, T, k, flat):
    # one expert to the largest expert count (the per-wave count table of
    # the fused routing fills the token buffer at E = 1024), E not a
    # multiple of the scan's experts per thread, flat and grouped outputs
    wl = synth.Workload(f"fused-E{E}", E=E, T=T, k=k, proj=(("w", 64, 128),), outliers=False,
                        bias="gauss", seed=1200 + E, swiglu=False)
    print(f"[E={E} T={T} k={k} flat={flat}] fused route + GEMM", flush=True)
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0))
    x = synth.tokens(wl).cuda()
    ids_d = torch.from_numpy(ids).cuda()
    epi = lib.EPI_NONE | (lib.OUT_FLAT if flat else 0)
    if flat:
        y1, off1, perm1, inv1 = lib.route_grouped_spgemm(ids_d, x, k, w, epi)
        off2, perm2, inv2 = lib.route(ids_d, E, k)
        y2 = lib.grouped_spgemm_gather(x, perm2, k, off2, w, epi)
        torch.cuda.synchronize()
        assert torch.equal(off1, off2) and torch.equal(inv1, inv2)
        assert torch.equal(perm1, perm2) and torch.equal(y1, y2)
    else:
        _same(lib, ids_d, x, k, w, epi, wl.name)
    bad = ids_d.clone()
    bad[0] = E          # dropped from the plan
    _same(lib, bad, x, k, w, lib.EPI_NONE, wl.name + " with an invalid id")


@pytest.mark.gpu
def test_fused_fallback_and_empty(lib):
    # tiny: T*k = 128 > 4E = 32 -> the call makes the two separate calls
    wl = synth.WORKLOADS["tiny"]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0))
    x = synth.tokens(wl).cuda()
    _same(lib, torch.from_numpy(ids).cuda(), x, wl.k, w, lib.EPI_NONE, "tiny (fallback)")
    # an empty batch leaves zero offsets
    y, off, perm, inv = lib.route_grouped_spgemm(torch.empty(0, dtype=torch.int32, device="cuda"),
                                                 x[:0], wl.k, w)
    torch.cuda.synchronize()
    assert int(off.abs().sum().item()) == 0 and y.shape[0] == 0


@pytest.mark.gpu
@pytest.mark.parametrize("paired,tiled", [(False, False), (False, True), (True, True)])
def test_fused_against_oracle(lib, paired, tiled):
    """A decode batch (E=16, T=8, k=2, N=64, K=256) routed in the GEMM launch,
    and the same batch through the gather GEMM, against the float64 oracle;
    4:8 weights in the canonical and the tiled layout, paired weights tiled
    (the canonical paired layout is an exchange format the GEMM rejects)."""
    wl = synth.Workload("fused", E=16, T=8, k=2, proj=(("w", 64, 256),), outliers=True,
                        bias="gauss", seed=4242)
    ids, _ = synth.routing(wl)
    x = synth.tokens(wl)
    w = pack_workload(lib, wl, 0, paired=paired)
    if tiled:
        w = lib.tile_weights(w)
    y, off, perm, inv = lib.route_grouped_spgemm(torch.from_numpy(ids).cuda(), x.cuda(), wl.k, w)
    yg = lib.grouped_spgemm_gather(x.cuda(), perm, wl.k, off, w)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    assert np.array_equal(off.cpu().numpy(), off_r)
    assert np.array_equal(perm.cpu().numpy(), perm_r)
    assert np.array_equal(inv.cpu().numpy(), inv_r)
    dec = [oracle_decode(oracle_expert(wl, 0, e, paired=paired)) for e in range(wl.E)]
    y_ref = oracle.grouped_gemm(oracle.permute(x.to(torch.float64).numpy(), perm_r, wl.k), off_r,
                                lambda e: dec[e])
    tol_check(f64(y), y_ref, f"fused decode batch, paired={paired}, tiled={tiled}")
    tol_check(f64(yg), y_ref, f"gather GEMM, paired={paired}, tiled={tiled}")


@pytest.mark.gpu
def test_gather_canonical_prefill_against_oracle(lib):
    """The gather GEMM on canonical (untiled) 4:8 weights over a batch with
    more than 32 rows per expert on average (the contraction tile), with
    SwiGLU, against the oracle."""
    wl = synth.Workload("gather-canonical", E=4, T=96, k=2, proj=(("w", 128, 320),),
                        outliers=True, bias="gauss", seed=4343)
    ids, _ = synth.routing(wl)
    x = synth.tokens(wl)
    w = pack_workload(lib, wl, 0)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    y = lib.grouped_spgemm_gather(x.cuda(), perm, wl.k, off, w, lib.EPI_SWIGLU)
    torch.cuda.synchronize()
    off_r, perm_r, _ = oracle.route(ids, wl.E)
    dec = [oracle_decode(oracle_expert(wl, 0, e)) for e in range(wl.E)]
    y_ref = oracle.grouped_gemm(oracle.permute(x.to(torch.float64).numpy(), perm_r, wl.k), off_r,
                                lambda e: dec[e])
    tol_check(f64(y), oracle.bf16_round(oracle.swiglu(y_ref)), "gather GEMM, canonical, SwiGLU")


@pytest.mark.gpu
def test_fused_in_graph(lib):
    """The fused call captured in a HIP graph: every replay, with eager work
    between replays, gives the eager result."""
    wl = synth.WORKLOADS["decode-30b"]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0))
    x = synth.tokens(wl).cuda()
    ids_d = torch.from_numpy(ids).cuda()
    want = lib.route_grouped_spgemm(ids_d, x, wl.k, w)
    outs = [torch.empty_like(t) for t in want]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.moesq_route_grouped_spgemm(ids_d, x, wl.T, wl.k, w, lib.EPI_NONE, outs[0], outs[1],
                                       outs[2], outs[3])
    rows = int(want[1][-1].item())
    for rep in range(3):
        for t in outs:
            t.zero_()
        lib.route(ids_d, wl.E, wl.k)              # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[1], want[1]), rep
        assert torch.equal(outs[2][:rows], want[2][:rows]), rep
        assert torch.equal(outs[3], want[3]), rep
        assert torch.equal(outs[0][:rows], want[0][:rows]), rep
