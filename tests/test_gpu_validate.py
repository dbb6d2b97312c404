"""moesq_validate: zero violations on valid inputs, exact counts on planted
ones (ids, offsets, masks, scales, global scales), for both weight layouts."""
from __future__ import annotations

import pytest
import torch

import synth
from gpu_util import pack_workload


def _inputs(m):
    wl = synth.WORKLOADS["tiny"]
    dev = torch.device("cuda")
    ids = torch.from_numpy(synth.routing(wl)[0]).to(dev)
    off = torch.empty(wl.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(wl.M, dtype=torch.int32, device=dev)
    inv = torch.empty(wl.M, dtype=torch.int32, device=dev)
    m.moesq_route(ids, wl.T, wl.k, wl.E, off, perm, inv)
    w = pack_workload(m, wl, 0)
    return wl, ids, off, w


@pytest.mark.gpu
def test_validate_accepts_valid_inputs(lib):
    wl, ids, off, w = _inputs(lib)
    zero = dict.fromkeys(lib.VALIDATE_CHECKS, 0)
    assert lib.moesq_validate(ids, wl.T, wl.k, wl.E, off, w) == zero
    assert lib.moesq_validate(ids, wl.T, wl.k, wl.E, off, lib.tile_weights(w)) == zero
    assert lib.moesq_validate(w=w) == zero                                  # weights only
    assert lib.moesq_validate(ids, wl.T, wl.k, wl.E) == zero                # ids only


@pytest.mark.gpu
@pytest.mark.parametrize("tiled", [False, True])
def test_validate_counts_planted_violations(lib, tiled):
    m = lib
    wl, ids, off, w = _inputs(m)
    ids = ids.clone()
    ids[[0, 5, 17]] = torch.tensor([-1, wl.E, wl.E + 5], dtype=torch.int32, device=ids.device)
    off = off.clone()
    off[wl.E] += 1                                   # offsets[E] != T*k
    masks = w.masks.clone()
    flat = masks.view(-1)
    flat[[3, 100, flat.numel() - 1]] = torch.tensor([0x07, 0x1F, 0x00], dtype=torch.uint8,
                                                   device=flat.device)   # 3, 5 and 0 bits
    scales = w.scales.clone()
    sf = scales.view(-1)
    sf[[2, sf.numel() - 3]] = torch.tensor([0x7F, 0x81], dtype=torch.uint8, device=sf.device)
    g = w.global_scale.clone()
    g[1] = float("nan")
    bad = m.Weights(w.values, masks, scales, g)
    if tiled:
        bad = m.tile_weights(bad)                   # shares the planted global scales
    counts = m.moesq_validate(ids, wl.T, wl.k, wl.E, off, bad)
    assert counts == {"ids": 3, "offsets": 1, "masks": 3, "scales": 2, "global_scales": 1}
    detail = m._last_error().decode()
    for word in ("ids", "offset", "masks", "scale", "global"):
        assert word in detail, detail


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16 * 7, 64 << 20])
def test_stream_read_runs(lib, nbytes):
    """The measurement read leaves the sink alone for data whose word XOR is
    not its marker (all-ones bytes XOR to 0 or 0x01010101), at ragged sizes."""
    m = lib
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.moesq_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
