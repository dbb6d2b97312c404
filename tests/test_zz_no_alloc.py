"""moesq_route_noalloc (routing without a workspace, for callers that cannot
allocate) through the C ABI: the same plan as moesq_route with a caller's
workspace, bit for bit, and as the oracle, on two calls in a row (the second
with fewer ids, so stale counts of the first would show), inside a captured
HIP graph, and the host rejection of inputs beyond the library's scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _plan(lib, ids, E, k, noalloc):
    M = ids.numel()
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    if noalloc:
        lib.moesq_route_noalloc(ids, M // k, k, E, off, perm, inv)
    else:
        nws = lib.moesq_route_workspace_bytes(M // k, k, E)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        lib.moesq_route(ids, M // k, k, E, off, perm, inv, ws)
    return off, perm, inv


def _ids(E, M, seed):
    rng = np.random.default_rng(seed)
    ids = np.minimum(rng.zipf(1.3, M) - 1, E - 1).astype(np.int32)
    return ids


@pytest.mark.parametrize("E,k,M1,M2", [
    (384, 8, 65536, 4104),       # both through the block kernels (scratch), second smaller
    (1024, 2, 300000, 70000),
    (128, 8, 32768, 128),        # second small enough for the one-workgroup path
    (384, 8, 1397760, 524288),   # the largest id count the scratch holds at E = 384
])
def test_noalloc_matches_workspace_route(lib, E, k, M1, M2):
    print(f"[noalloc] E={E} k={k} M={M1} then M={M2}", flush=True)
    for M, seed in [(M1, E + M1), (M2, E + M2)]:
        ids_np = _ids(E, M, seed)
        ids = torch.from_numpy(ids_np).cuda()
        got = _plan(lib, ids, E, k, noalloc=True)
        want = _plan(lib, ids, E, k, noalloc=False)
        torch.cuda.synchronize()
        ref = oracle.route(ids_np, E)
        for g, w_, r, what in zip(got, want, ref, ("offsets", "perm", "inv_perm")):
            assert torch.equal(g, w_), f"E={E} M={M}: {what} differs from moesq_route"
            assert np.array_equal(g.cpu().numpy(), r), f"E={E} M={M}: {what} differs from the oracle"


def test_noalloc_rejects_beyond_scratch(lib):
    """Block counts beyond the scratch: an error on the host, nothing launched."""
    E, k = 1024, 1
    M = 524288 + 512                  # one block more than the scratch holds at E = 1024
    assert lib.moesq_route_workspace_bytes(M, k, E) > lib.ROUTE_SCRATCH_BYTES
    ids = torch.zeros(M, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(M, dtype=torch.int32, device="cuda")
    inv = torch.empty(M, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.MoesqError) as ei:
        lib.moesq_route_noalloc(ids, M, k, E, off, perm, inv)
    assert ei.value.status == lib.ERR_SHAPE
    assert "scratch" in str(ei.value)
    # one block less fits
    M = 524288
    lib.moesq_route_noalloc(ids[:M], M, k, E, off, perm[:M], inv[:M])
    torch.cuda.synchronize()
    assert int(off[1].item()) == M


def test_noalloc_in_graph(lib):
    """Captured in a HIP graph (where allocation is not allowed) and replayed
    three times with eager routing of other ids in between: every replay
    gives the eager plan."""
    E, k, M = 384, 8, 65536
    ids_np = _ids(E, M, 5)
    ids = torch.from_numpy(ids_np).cuda()
    want = _plan(lib, ids, E, k, noalloc=False)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(M, dtype=torch.int32, device="cuda")
    inv = torch.empty(M, dtype=torch.int32, device="cuda")
    other = torch.from_numpy(_ids(E, M, 6)).cuda()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.moesq_route_noalloc(ids, M // k, k, E, off, perm, inv)
    for rep in range(3):
        _plan(lib, other, E, k, noalloc=True)      # eager work on the same scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(off, want[0]) and torch.equal(perm, want[1]), rep
        assert torch.equal(inv, want[2]), rep
