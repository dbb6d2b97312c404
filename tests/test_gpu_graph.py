"""The hot path captured in a HIP graph replays to the eager result.

A serving step (and bench.py) replays the chain route -> permute -> grouped
GEMM (SwiGLU) -> grouped GEMM -> weighted combine as one HIP graph.  Each
case captures the chain once, then replays it three times with eager work
(clearing the outputs) and a device synchronisation between replays, and
checks every replay bit for bit against the eager run.  The second case has
more than 4096 routed rows, so routing takes the multi-workgroup path with
its workspace.
"""
from __future__ import annotations

import pytest
import torch

import synth
from gpu_util import pack_workload

CASES = [
    synth.Workload("graph-decode", E=32, T=64, k=8, proj=(("gate_up", 256, 256), ("down", 128, 128)),
                   outliers=True, bias="gauss", seed=1101, swiglu=True, weighted_combine=True),
    synth.Workload("graph-prefill", E=16, T=1024, k=8, proj=(("gate_up", 128, 128), ("down", 64, 64)),
                   outliers=True, bias="zipf", seed=1102, swiglu=True, weighted_combine=True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_graph_replays_match_eager(lib, wl):
    m = lib
    dev = torch.device("cuda")
    ids, tw = synth.routing(wl)
    ids = torch.from_numpy(ids).to(dev)
    tw = torch.from_numpy(tw).to(dev)
    x = synth.tokens(wl).to(dev)
    w = [m.tile_weights(pack_workload(m, wl, p)) for p in range(2)]
    E, T, k, M = wl.E, wl.T, wl.k, wl.M
    i32 = dict(dtype=torch.int32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    off, perm, inv = torch.empty(E + 1, **i32), torch.empty(M, **i32), torch.empty(M, **i32)
    nws = m.moesq_route_workspace_bytes(T, k, E)
    assert (nws > 0) == (M > 4096)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    xr = torch.empty(M, wl.K_in, **bf)
    h = torch.empty(M, wl.proj[0][1] // 2, **bf)
    y = torch.empty(M, wl.proj[1][1], **bf)
    out = torch.empty(T, wl.proj[1][1], **bf)

    def chain():
        m.moesq_route(ids, T, k, E, off, perm, inv, ws)
        m.moesq_permute(x, perm, T, k, wl.K_in, xr)
        m.moesq_grouped_spgemm(xr, off, M, w[0], m.EPI_SWIGLU, h)
        m.moesq_grouped_spgemm(h, off, M, w[1], m.EPI_NONE, y)
        m.moesq_unpermute(y, inv, tw, T, k, wl.proj[1][1], out)

    chain()
    torch.cuda.synchronize()
    want = [t.clone() for t in (off, perm, inv, h, out)]
    assert torch.isfinite(want[-1].float()).all()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for r in range(3):
        for t in (off, perm, inv):
            t.fill_(-7)
        for t in (xr, h, y, out):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("offsets", "perm", "inv_perm", "h", "out"),
                                  (off, perm, inv, h, out), want):
            assert torch.equal(got, ref), f"replay {r}: {name} differs from the eager run"


@pytest.mark.gpu
@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
def test_w4a4_graph_replays_match_eager(lib, paired):
    """The W4A4 chain (route -> quantize tokens -> gathered W4A4 gate/up with
    SwiGLU -> quantize h -> W4A4 down -> weighted combine) in one graph."""
    m = lib
    wl = CASES[1]
    dev = torch.device("cuda")
    ids, tw = synth.routing(wl)
    ids = torch.from_numpy(ids).to(dev)
    tw = torch.from_numpy(tw).to(dev)
    x = synth.tokens(wl).to(dev)
    w = [m.tile_weights(pack_workload(m, wl, p, paired=paired)) for p in range(2)]
    E, T, k, M = wl.E, wl.T, wl.k, wl.M
    i32 = dict(dtype=torch.int32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    off, perm, inv = torch.empty(E + 1, **i32), torch.empty(M, **i32), torch.empty(M, **i32)
    nws = m.moesq_route_workspace_bytes(T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    xq = m.Act4.empty(T, wl.K_in)
    hq = m.Act4.empty(M, wl.proj[0][1] // 2)
    h = torch.empty(M, wl.proj[0][1] // 2, **bf)
    y = torch.empty(M, wl.proj[1][1], **bf)
    out = torch.empty(T, wl.proj[1][1], **bf)

    def chain():
        m.moesq_route(ids, T, k, E, off, perm, inv, ws)
        m.moesq_quantize_activations(x, T, wl.K_in, xq.codes, xq.scales, xq.row_scale)
        m.moesq_grouped_spgemm_act4(xq, perm, T, k, off, M, w[0], m.EPI_SWIGLU, h)
        m.moesq_quantize_activations(h, M, h.shape[1], hq.codes, hq.scales, hq.row_scale)
        m.moesq_grouped_spgemm_act4(hq, None, 0, 1, off, M, w[1], m.EPI_NONE, y)
        m.moesq_unpermute(y, inv, tw, T, k, wl.proj[1][1], out)

    chain()
    torch.cuda.synchronize()
    want = [t.clone() for t in (off, perm, xq.codes, xq.scales, h, hq.codes, out)]
    assert torch.isfinite(want[-1].float()).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for r in range(3):
        for t in (off, perm, inv):
            t.fill_(-7)
        for t in (xq.codes, xq.scales, hq.codes, hq.scales):
            t.fill_(0xAA)
        for t in (h, y, out):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("offsets", "perm", "token codes", "token scales", "h",
                                   "h codes", "out"),
                                  (off, perm, xq.codes, xq.scales, h, hq.codes, out), want):
            assert torch.equal(got, ref), f"W4A4 replay {r}: {name} differs from the eager run"
