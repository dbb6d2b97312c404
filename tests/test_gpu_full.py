"""Full-tensor parity on the tiny and 30B-class workloads (E=8, T=64, k=2,
N=128, K=256; E=128, N=1536, K=2048 with T=16 or T=4096, k=8), both weight
formats: every output element against the float64 oracle, per tensor
(relative Frobenius error and max abs error), in the launch configuration the
benchmark times (routing and scatter fused into the GEMM on decode batches,
the gather GEMM with the flat-order epilogue otherwise) and through the plain
calls (route, permute, GEMM in routed order, weighted combine).  The oracle
compresses every active expert itself from the same dense weights."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_same_pack, f64, oracle_experts, pack_workload, tol_check

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
@pytest.mark.parametrize("name", ["tiny", "decode-30b", "prefill-30b"])
def test_full_tensor(lib, name, paired):
    wl = synth.WORKLOADS[name]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    say(f"[{name}] paired={paired}: packing {wl.E} experts on the GPU")
    wc = pack_workload(lib, wl, 0, paired=paired)
    w = lib.tile_weights(wc)
    xd, ids_d = x.cuda(), torch.from_numpy(ids).cuda()
    # the benchmark's launch configuration
    decode_batch = wl.M <= 1024 and wl.M <= 4 * wl.E
    if decode_batch:
        flat, off_b, perm_b, inv_b = lib.route_grouped_spgemm(ids_d, xd, wl.k, w,
                                                              lib.EPI_NONE | lib.OUT_FLAT)
    else:
        off_b, perm_b, inv_b = lib.route(ids_d, wl.E, wl.k)
        flat = lib.grouped_spgemm_gather(xd, perm_b, wl.k, off_b, w, lib.EPI_NONE | lib.OUT_FLAT)
    # the plain calls
    off, perm, inv = lib.route(ids_d, wl.E, wl.k)
    y = lib.grouped_spgemm(lib.permute(xd, perm, wl.k), off, w)
    out = lib.unpermute(y, inv, torch.from_numpy(tw).cuda(), wl.T, wl.k)
    torch.cuda.synchronize()

    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    for got, what in [((off_b, perm_b, inv_b), "fused plan"), ((off, perm, inv), "plan")]:
        for a, b, part in zip(got, (off_r, perm_r, inv_r), ("offsets", "perm", "inv_perm")):
            assert np.array_equal(a.cpu().numpy(), b), f"{name} {what}: {part} differs"
    active = np.nonzero(np.diff(off_r))[0]
    say(f"[{name}] oracle compresses {len(active)} active experts")
    ref = oracle_experts(wl, 0, active, paired=paired)
    for e in active:
        assert_same_pack(wc, int(e), ref[int(e)][0], f"{name} expert {e}")
    x64 = x.to(torch.float64).numpy()
    y_ref = oracle.grouped_gemm(oracle.permute(x64, perm_r, wl.k), off_r,
                                lambda e: ref[int(e)][1])
    rel, mx = tol_check(f64(y), y_ref, f"{name} Y (routed order)")
    say(f"[{name}] Y: rel Frobenius {rel:.2e}, max abs {mx:.2e}")
    tol_check(f64(flat), oracle.unpermute(y_ref, inv_r, None, wl.T, wl.k),
              f"{name} Y (flat order, benchmark launch)")
    tol_check(f64(out), oracle.unpermute(y_ref, inv_r, tw, wl.T, wl.k),
              f"{name} weighted combine")
    say(f"[{name}] paired={paired}: every output element within tolerance")
