"""Parity of the HIP path (through the C ABI) with the CPU oracle on the
same seeded inputs.  Integer and byte results are bit-exact; bf16 outputs
meet the relative-Frobenius / max-abs tolerance of gpu_util.tol_check.

Run on an MI355X: python -u -m pytest tests -m gpu -x -v"""
import itertools
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_same_pack, f64, oracle_expert, oracle_experts, pack_workload,
                      pick_experts, tol_check)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _route_ref(ids, E):
    return oracle.route(ids, E)


def _gpu_route(m, ids_np, E, k):
    ids = torch.from_numpy(ids_np).cuda()
    off, perm, inv = m.route(ids, E, k)
    torch.cuda.synchronize()
    return off.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy()


# ------------------------------------------------------------------ packing

def test_pack_golden_rows(lib):
    """The GPU packer reproduces the hand-derived fixture bytes."""
    import pins
    d = {ln[0]: ln[1:] for ln in pins._lines("quant_rows.txt")}
    W = torch.tensor([[float(v) for v in d["w0"]], [float(v) for v in d["w1"]]],
                     dtype=torch.float32).reshape(1, 2, 64).cuda()
    w = lib.pack_weights(W)
    torch.cuda.synchronize()
    for r in range(2):
        assert w.masks[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"masks{r}"]]
        assert w.values[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"values{r}"]]
        assert w.scales[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"scales{r}"]]
    assert w.global_scale[0].item() == float(d["g"][0])


def test_pack_and_decode_tiny(lib):
    wl = synth.WORKLOADS["tiny"]
    dense = synth.dense_experts(wl, 0)                      # CPU draw, same tensor both sides
    w = lib.pack_weights(dense.cuda())
    torch.cuda.synchronize()
    for e in range(wl.E):
        p = oracle.quantize(dense[e].numpy())
        assert_same_pack(w, e, p, f"expert {e}")
        dec = lib.decode_weights(w, e)
        torch.cuda.synchronize()
        assert np.array_equal(f64(dec), oracle.decode(p, include_global=False)), e


def test_pack_extreme_ranges(lib):
    """Subnormal and zero block scales, saturating values, ties, all-zero rows
    and an all-zero expert."""
    g = torch.Generator().manual_seed(11)
    E, N, K = 3, 32, 256
    d = torch.randn(E, N, K, generator=g)
    d[0] *= torch.pow(10.0, torch.empty(N, 1).uniform_(-9, 1, generator=g))   # per-row range
    d[0, 3] = 0.0                                                            # zero row
    d[0, 4, :64] = 0.25                                                      # all-equal groups
    d[1, :, ::7] *= 300.0                                                    # strong outliers
    d[2] = 0.0                                                               # zero expert
    w = lib.pack_weights(d.cuda())
    torch.cuda.synchronize()
    for e in range(E):
        p = oracle.quantize(d[e].numpy())
        assert_same_pack(w, e, p, f"expert {e}")
        assert np.array_equal(f64(lib.decode_weights(w, e)), oracle.decode(p, include_global=False))


def _tiled_ref(arr, nbytes_per_seg):
    """The tiled permutation written from its definition: [E][N][K/X] ->
    [E][N/32][K/64][32][bytes per 64-position segment]."""
    E, N, W = arr.shape
    J = W // nbytes_per_seg
    return arr.reshape(E, N // 32, 32, J, nbytes_per_seg).transpose(0, 1, 3, 2, 4).reshape(E, N, W)


def test_tile_layout_and_decode(lib):
    g = torch.Generator().manual_seed(5)
    E, N, K = 3, 96, 448
    d = torch.randn(E, N, K, generator=g) * 0.02
    w = lib.pack_weights(d.cuda())
    t = lib.tile_weights(w)
    torch.cuda.synchronize()
    for name, seg in [("values", 16), ("masks", 8), ("scales", 2)]:
        a = getattr(w, name).cpu().numpy()
        b = getattr(t, name).cpu().numpy()
        assert np.array_equal(b, _tiled_ref(a, seg)), name
    for e in range(E):
        p = oracle.quantize(d[e].numpy())
        assert np.array_equal(f64(lib.decode_weights(t, e)), oracle.decode(p, include_global=False))


def test_tile_rejects_shapes(lib):
    w = lib.pack_weights(torch.zeros(1, 48, 64, device="cuda"))
    with pytest.raises(lib.MoesqError):
        lib.tile_weights(w)                       # N % 32 != 0
    w = lib.pack_weights(torch.zeros(1, 64, 96, device="cuda"))
    with pytest.raises(lib.MoesqError):
        lib.tile_weights(w)                       # K % 64 != 0


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_route_workloads(lib, name):
    wl = synth.WORKLOADS[name]
    ids, _ = synth.routing(wl)
    got = _gpu_route(lib, ids, wl.E, wl.k)
    ref = _route_ref(ids, wl.E)
    for a, b, what in zip(got, ref, ["offsets", "perm", "inv_perm"]):
        assert np.array_equal(a, b), f"{name}: {what} differs"


@pytest.mark.parametrize("E,M,k,mode", [
    (1, 64, 1, "random"), (8, 1, 1, "random"), (8, 640, 4, "same"), (1024, 70000, 2, "random"),
    (384, 65536, 8, "skew"), (5, 63, 3, "random"), (2, 129, 1, "random"),
    (384, 1000008, 8, "skew")])   # 1954 blocks: a partial batch of block counts and a partial last block
def test_route_edges(lib, E, M, k, mode):
    rng = np.random.default_rng(E * 7 + M)
    if mode == "same":
        ids = np.full(M, E - 1, np.int32)
    elif mode == "skew":
        ids = np.minimum(rng.zipf(1.3, M) - 1, E - 1).astype(np.int32)
    else:
        ids = rng.integers(0, E, M).astype(np.int32)
    got = _gpu_route(lib, ids, E, k)
    ref = _route_ref(ids, E)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("E,M", [(384, 65536), (1024, 70001), (7, 5000)])
def test_route_single_workgroup_path(lib, E, M):
    """Without workspace, large inputs take the one-workgroup path."""
    rng = np.random.default_rng(M)
    ids = rng.integers(0, E, M).astype(np.int32)
    d = torch.from_numpy(ids).cuda()
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(M, dtype=torch.int32, device="cuda")
    inv = torch.empty(M, dtype=torch.int32, device="cuda")
    lib.moesq_route(d, M, 1, E, off, perm, inv, None)
    torch.cuda.synchronize()
    ref = oracle.route(ids, E)
    for a, b in zip((off, perm, inv), ref):
        assert np.array_equal(a.cpu().numpy(), b)


@pytest.mark.parametrize("big", [False, True])
def test_route_invalid_ids(lib, big):
    E, k = 6, 2
    ids = np.array([0, 5, -1, 3, 6, 3, 1000, 0, 2, 5], np.int32)
    if big:
        ids = np.tile(ids, 1000)
    off, perm, inv = _gpu_route(lib, ids, E, k)
    valid = (ids >= 0) & (ids < E)
    vidx = np.nonzero(valid)[0]
    o2, p2, _ = oracle.route(ids[valid], E)
    assert np.array_equal(off, o2)
    n = len(vidx)
    assert np.array_equal(perm[:n], vidx[p2])
    assert (inv[~valid] == -1).all()
    assert np.array_equal(inv[vidx[p2]], np.arange(n))


# ------------------------------------------------------------------ dispatch and combine

@pytest.mark.parametrize("name", ["tiny", "decode-1t", "prefill-30b"])
def test_permute(lib, name):
    wl = synth.WORKLOADS[name]
    ids, _ = synth.routing(wl)
    x = synth.tokens(wl)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    xr = lib.permute(x.cuda(), perm, wl.k)
    torch.cuda.synchronize()
    _, pref, _ = oracle.route(ids, wl.E)
    assert torch.equal(xr.cpu(), x[torch.from_numpy(pref.astype(np.int64)) // wl.k])


@pytest.mark.parametrize("T,k,N", [(64, 2, 128), (1024, 8, 7168), (5, 3, 8), (37, 10, 136)])
def test_unpermute(lib, T, k, N):
    E = max(k, 16)
    rng = np.random.default_rng(T + N)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).reshape(-1).astype(np.int32)
    w = rng.random(T * k).astype(np.float32)
    g = torch.Generator().manual_seed(T * N)
    y = torch.randn(T * k, N, generator=g).to(torch.bfloat16)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, k)
    yd = y.cuda()
    out_w = lib.unpermute(yd, inv, torch.from_numpy(w).cuda(), T, k)
    out_f = lib.unpermute(yd, inv, None, T, k)
    torch.cuda.synchronize()
    _, _, inv_ref = oracle.route(ids, E)
    y64 = y.to(torch.float64).numpy()
    tol_check(f64(out_w), oracle.unpermute(y64, inv_ref, w, T, k), "weighted combine")
    assert np.array_equal(f64(out_f), oracle.unpermute(y64, inv_ref, None, T, k))


# ------------------------------------------------------------------ grouped GEMM

def _full_oracle_gemm(ids, E, k, x, packs, swiglu=False, packs2=None, weights=None):
    off, perm, inv = oracle.route(ids, E)
    dec = [oracle.decode(p) for p in packs]
    xr = oracle.permute(x.to(torch.float64).numpy(), perm, k)
    y = oracle.grouped_gemm(xr, off, lambda e: dec[e])
    return off, perm, inv, y


@pytest.mark.parametrize("tiled", [False, True])
def test_spgemm_tiny_end_to_end(lib, tiled):
    """tiny: route -> permute -> GEMM -> flat and weighted combine, every
    output against the oracle."""
    wl = synth.WORKLOADS["tiny"]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    dense = synth.dense_experts(wl, 0)
    packs = [oracle.quantize(dense[e].numpy()) for e in range(wl.E)]
    w = lib.pack_weights(dense.cuda())
    if tiled:
        w = lib.tile_weights(w)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    xr = lib.permute(x.cuda(), perm, wl.k)
    y = lib.grouped_spgemm(xr, off, w)
    out = lib.unpermute(y, inv, torch.from_numpy(tw).cuda(), wl.T, wl.k)
    flat = lib.unpermute(y, inv, None, wl.T, wl.k)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r, y_ref = _full_oracle_gemm(ids, wl.E, wl.k, x, packs)
    tol_check(f64(y), y_ref, "Y")
    tol_check(f64(flat), oracle.unpermute(y_ref, inv_r, None, wl.T, wl.k), "flat combine")
    tol_check(f64(out), oracle.unpermute(y_ref, inv_r, tw, wl.T, wl.k), "weighted combine")


def _edge_case(lib, loads, N, K, swiglu, seed, tiled=False):
    E = len(loads)
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    rng = np.random.default_rng(seed)
    ids = ids[rng.permutation(len(ids))]
    M = len(ids)
    wl = synth.Workload("edge", E=E, T=M, k=1, proj=(("w", N, K),), outliers=True,
                        bias="none", seed=seed)
    x = synth.tokens(wl, T=M, K=K)
    dense = synth.dense_experts(wl, 0)
    packs = [oracle.quantize(dense[e].numpy()) for e in range(E)]
    w = lib.pack_weights(dense.cuda())
    if tiled:
        w = lib.tile_weights(w)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, 1)
    xr = lib.permute(x.cuda(), perm, 1)
    y = lib.grouped_spgemm(xr, off, w, lib.EPI_SWIGLU if swiglu else lib.EPI_NONE)
    torch.cuda.synchronize()
    _, _, _, y_ref = _full_oracle_gemm(ids, E, 1, x, packs)
    if swiglu:
        y_ref = oracle.bf16_round(oracle.swiglu(y_ref))
    tol_check(f64(y), y_ref, f"loads={loads} N={N} K={K} swiglu={swiglu} tiled={tiled}")


@pytest.mark.parametrize("loads,N,K,swiglu", [
    ([0, 1, 15, 16, 17, 33, 130, 0], 64, 96, False),
    ([0, 1, 15, 16, 17, 33, 130, 0], 64, 96, True),
    ([300], 48, 32, False),
    ([0, 0, 0, 200, 0], 272, 160, False),
    ([0, 0, 0, 200, 0], 288, 160, True),
    ([5, 0, 64, 127, 128, 129, 1], 16, 416, False),
    ([1] * 20, 128, 256, True),
])
def test_spgemm_edges(lib, loads, N, K, swiglu):
    _edge_case(lib, loads, N, K, swiglu, seed=sum(loads) + N + K)


@pytest.mark.parametrize("loads,N,K,swiglu", [
    ([0, 1, 15, 16, 17, 33, 130, 0], 64, 128, False),
    ([0, 1, 15, 16, 17, 33, 130, 0], 128, 192, True),
    ([0, 0, 0, 200, 0], 288, 320, False),
    ([5, 0, 64, 127, 128, 129, 1], 32, 448, False),
    ([1] * 20, 128, 256, True),
    ([40] * 4, 64, 64, False),
    # tile choice of a short call (one launch): M = 4E the one-fragment
    # streaming tile (an expert of 20 rows takes two token tiles); up to 32
    # rows per expert on average the two-fragment streaming tile, above it
    # the contraction tile
    ([20, 0, 10, 2, 0, 0, 0, 0], 64, 512, False),
    ([20, 1, 10, 2, 0, 0, 0, 0], 64, 512, True),
    ([80, 0, 40, 8], 128, 512, False),
    ([80, 1, 40, 8], 128, 512, True),
    # the largest expert count: 1024 experts of 0-2 rows
    ([(i * 7) % 3 for i in range(1024)], 32, 64, False),
])
def test_spgemm_edges_tiled(lib, loads, N, K, swiglu):
    _edge_case(lib, loads, N, K, swiglu, seed=sum(loads) + N + K + 1, tiled=True)


@pytest.mark.parametrize("name,swiglu", [("tiny", False), ("decode-30b", False),
                                         ("prefill-30b", False), ("decode-1t", True)])
def test_spgemm_gather_matches_permute(lib, name, swiglu):
    """Dispatch fused into the GEMM gives the bytes of permute + GEMM, also
    where the permutation has out-of-range entries (zero rows)."""
    wl = synth.WORKLOADS[name]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    x = synth.tokens(wl).cuda()
    epi = lib.EPI_SWIGLU if swiglu else lib.EPI_NONE
    want = lib.grouped_spgemm(lib.permute(x, perm, wl.k), off, w, epi)
    got = lib.grouped_spgemm_gather(x, perm, wl.k, off, w, epi)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    bad = perm.clone()
    bad[[0, wl.M // 2, wl.M - 1]] = torch.tensor([-1, wl.M, 1 << 30], dtype=torch.int32, device=bad.device)
    want = lib.grouped_spgemm(lib.permute(x, bad, wl.k), off, w, epi)
    got = lib.grouped_spgemm_gather(x, bad, wl.k, off, w, epi)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert not got[[0, wl.M // 2, wl.M - 1]].any()


def _split_launch_case(lib, paired, swiglu):
    """A call of at least 5.5e11 multiply-adds: the library splits the experts
    over three launches by their own row counts (up to 16, 17-32, more).
    Experts of 9, 16, 17, 25, 32, 33 and 65,468 rows cover every launch and
    both sides of each boundary; every row of the small experts and 256 rows
    of the large one are checked against the oracle."""
    loads = [9, 16, 17, 25, 32, 33, 65468]
    N, K = 2048, 4096
    M = sum(loads)
    assert M * N * K >= 5.5e11
    E = len(loads)
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    ids = ids[np.random.default_rng(77).permutation(M)]
    wl = synth.Workload("split", E=E, T=M, k=1, proj=(("w", N, K),), outliers=True,
                        bias="none", seed=4242)
    x = synth.tokens(wl, T=M, K=K)
    say(f"[split launches] paired={paired} swiglu={swiglu}: packing {E} experts {N}x{K}")
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, 1)
    y = lib.grouped_spgemm_gather(x.cuda(), perm, 1, off, w,
                                  lib.EPI_SWIGLU if swiglu else lib.EPI_NONE)
    torch.cuda.synchronize()
    off_r, perm_r, _ = oracle.route(ids, E)
    x64 = x.to(torch.float64).numpy()
    ref = oracle_experts(wl, 0, range(E), paired=paired)
    for e in range(E):
        rows = np.arange(off_r[e], off_r[e + 1])
        if len(rows) > 256:
            rows = np.concatenate([rows[:128], rows[-128:]])
        want = oracle.expert_gemm(x64[perm_r[rows]], ref[e][1])
        if swiglu:
            want = oracle.bf16_round(oracle.swiglu(want))
        tol_check(f64(y[torch.from_numpy(rows).cuda()]), want,
                  f"split launches paired={paired} swiglu={swiglu} expert {e} ({loads[e]} rows)")
    say(f"[split launches] paired={paired} swiglu={swiglu} ok")


@pytest.mark.parametrize("paired,swiglu", [(False, False), (False, True), (True, False),
                                           (True, True)])
def test_spgemm_split_launches(lib, paired, swiglu):
    _split_launch_case(lib, paired, swiglu)


@pytest.mark.parametrize("name", ["decode-1t", "prefill-1t"])
def test_chain_1t_workloads(lib, name):
    """Full-size trillion-class chain in the benchmark's launch configuration:
    dispatch fused into the gate/up GEMM with SwiGLU -> down GEMM -> combine.
    Sampled experts (the largest, one from each launch range of row counts
    and a random one): packed bytes and every h and Y2 row against the oracle
    chain.  The combine at full size against the oracle's combine of the
    device's Y2 (float64 on the host)."""
    wl = synth.WORKLOADS[name]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    say(f"[{name}] packing 2 x {wl.E} experts on the GPU")
    w1 = pack_workload(lib, wl, 0)
    w2 = pack_workload(lib, wl, 1)
    w1t, w2t = lib.tile_weights(w1), lib.tile_weights(w2)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    say(f"[{name}] chain M={wl.M} (tiled weights, dispatch fused into the gate/up GEMM)")
    h = lib.grouped_spgemm_gather(x.cuda(), perm, wl.k, off, w1t, lib.EPI_SWIGLU)
    y2 = lib.grouped_spgemm(h, off, w2t)
    tw_d = torch.from_numpy(tw).cuda()
    out = lib.unpermute(y2, inv, tw_d if wl.weighted_combine else None, wl.T, wl.k)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    counts = np.diff(off_r)
    x64 = x.to(torch.float64).numpy()
    rng = np.random.default_rng(wl.seed)
    picks = pick_experts(counts, rng)
    say(f"[{name}] oracle for experts {picks} (rows {[int(counts[e]) for e in picks]})")
    ref1 = oracle_experts(wl, 0, picks)
    ref2 = oracle_experts(wl, 1, picks)
    for e in picks:
        assert_same_pack(w1, e, ref1[e][0], f"{name} gate_up expert {e}")
        assert_same_pack(w2, e, ref2[e][0], f"{name} down expert {e}")
        rows = np.arange(off_r[e], off_r[e + 1])
        y1_ref = oracle.expert_gemm(x64[perm_r[rows] // wl.k], ref1[e][1])
        h_ref = oracle.bf16_round(oracle.swiglu(y1_ref))
        y2_ref = oracle.expert_gemm(h_ref, ref2[e][1])
        rows_t = torch.from_numpy(rows).cuda()
        tol_check(f64(h[rows_t]), h_ref, f"{name} h, expert {e}")
        tol_check(f64(y2[rows_t]), y2_ref, f"{name} Y2, expert {e}")
        say(f"[{name}] expert {e}: {counts[e]} rows ok")
    y2_host = f64(y2)
    want = oracle.unpermute(y2_host, inv_r, tw if wl.weighted_combine else None, wl.T, wl.k)
    if wl.weighted_combine:
        tol_check(f64(out), want, f"{name} weighted combine")
    else:
        assert np.array_equal(f64(out), want)
    say(f"[{name}] combine ok")
