"""Paired 4:8 weights through the C ABI against the CPU oracle: the GPU
packer's bytes (bit-exact), the tiled layout, decode (bit-exact) and the
sparse-MFMA grouped GEMM on both tiles, with SwiGLU, fused dispatch, ragged
tails and full-size sampled experts (bf16 tolerance of gpu_util.tol_check).

Format: paper summary page, "A Sparse-quantized representation" (Blackwell
paired 4:8 NVFP4, Storage layout)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_same_pack, f64, oracle_decode, oracle_expert, oracle_experts,
                      pack_workload, pick_experts, tol_check)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tiled(arr, seg):
    """[E][N][W] -> [E][N/32][W/seg][32][seg] (the segment tiling)."""
    E, N, W = arr.shape
    return arr.reshape(E, N // 32, 32, W // seg, seg).transpose(0, 1, 3, 2, 4).reshape(E, N, W)


def _paired_tiled_ref(values, patterns, scales):
    """The paired tiled layout written from its definition in moesq.h: per
    unit (groups G, G'), codes G v0, G v2, G' v0, G' v2, G v1, G v3, G' v1,
    G' v3 in nibbles 0..7 of a dword, and window byte w(G) | w(G') << 4 with
    w = i | j << 2 for the kept pairs i < j; then the segment tiling."""
    E, N, K4 = values.shape
    K = 4 * K4
    codes = np.stack([values & 15, values >> 4], -1).reshape(E, N, K // 8, 4).astype(np.uint32)
    pat = np.stack([patterns & 15, patterns >> 4], -1).reshape(E, N, K // 8)
    G, H = codes[:, :, 0::2], codes[:, :, 1::2]
    slots = [G[..., 0], G[..., 2], H[..., 0], H[..., 2], G[..., 1], G[..., 3], H[..., 1], H[..., 3]]
    dword = np.zeros(G.shape[:3], np.uint32)
    for i, c in enumerate(slots):
        dword |= c << np.uint32(4 * i)
    vbytes = dword.astype("<u4").view(np.uint8).reshape(E, N, K4)
    win = np.array([i | (j << 2) for i, j in oracle.PAIRS], np.uint8)
    wbytes = (win[pat[:, :, 0::2]] | (win[pat[:, :, 1::2]] << 4)).astype(np.uint8)
    return _tiled(vbytes, 16), _tiled(wbytes, 4), _tiled(scales, 2)


# ------------------------------------------------------------------ packing, tiling, decode

def test_paired_pack_golden_rows(lib):
    """The GPU packer reproduces the hand-derived paired fixture."""
    import pins
    d = {ln[0]: ln[1:] for ln in pins._lines("paired_rows.txt") if ln[0] != "pattern"}
    w0 = torch.tensor([float(v) for v in d["w0"]], dtype=torch.float32)
    W = torch.stack([w0, -w0]).reshape(1, 2, 32).cuda()
    w = lib.pack_weights(W, paired=True)
    torch.cuda.synchronize()
    for r in range(2):
        assert w.values[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"values{r}"]]
        assert w.masks[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d["patterns0"]]
        assert w.scales[0, r].cpu().numpy().tolist() == [int(t, 16) for t in d["scales0"]]
    assert w.global_scale[0].item() == float(d["g"][0])


def test_paired_pack_and_decode(lib):
    """Random, tie-heavy and extreme-range experts: packed bytes equal the
    oracle's; decode of the canonical and the tiled layout equals the
    oracle's decode (bf16 bit-exact); the tiled bytes equal the layout's
    definition."""
    g = torch.Generator().manual_seed(21)
    E, N, K = 4, 64, 448
    d = torch.randn(E, N, K, generator=g) * 0.02
    d[1] = torch.round(d[1] * 200) / 200                 # many equal pair sums
    d[1, 5, :64] = 0.5                                   # all pairs equal
    d[2] *= torch.pow(10.0, torch.empty(N, 1).uniform_(-9, 1, generator=g))
    d[2, 3] = 0.0
    d[3, :, ::5] *= 300.0                                # the largest weight often dropped
    w = lib.pack_weights(d.cuda(), paired=True)
    t = lib.tile_weights(w)
    torch.cuda.synchronize()
    assert t.layout == lib.LAYOUT_PAIRED_TILED
    for e in range(E):
        p = oracle.quantize_paired(d[e].numpy())
        assert_same_pack(w, e, p, f"expert {e}")
        want = oracle.decode_paired(p, include_global=False)
        assert np.array_equal(f64(lib.decode_weights(w, e)), want), e
        assert np.array_equal(f64(lib.decode_weights(t, e)), want), e
    rv, rw, rs = _paired_tiled_ref(w.values.cpu().numpy(), w.masks.cpu().numpy(),
                                   w.scales.cpu().numpy())
    assert np.array_equal(t.values.cpu().numpy(), rv)
    assert np.array_equal(t.masks.cpu().numpy(), rw)
    assert np.array_equal(t.scales.cpu().numpy(), rs)


def test_paired_validate(lib):
    """Valid paired weights pass; planted bad pattern nibbles are counted in
    both layouts."""
    g = torch.Generator().manual_seed(22)
    w = lib.pack_weights((torch.randn(2, 32, 128, generator=g) * 0.02).cuda(), paired=True)
    t = lib.tile_weights(w)
    zero = dict.fromkeys(lib.VALIDATE_CHECKS, 0)
    assert lib.moesq_validate(w=w) == zero
    assert lib.moesq_validate(w=t) == zero
    bad = w.masks.clone()
    bad.view(-1)[[0, 7, bad.numel() - 1]] = torch.tensor([0x06, 0x70, 0xFF], dtype=torch.uint8,
                                                       device=bad.device)
    counts = lib.moesq_validate(w=lib.Weights(w.values, bad, w.scales, w.global_scale,
                                              lib.LAYOUT_PAIRED))
    assert counts["masks"] == 3
    badt = t.masks.clone()
    badt.view(-1)[[1, 9]] = torch.tensor([0x44, 0x4C], dtype=torch.uint8, device=badt.device)
    badt.view(-1)[2] = 0x5E                         # 5: positions (1, 1), not a pair couple
    badt.view(-1)[3] = 0x84                         # valid
    counts = lib.moesq_validate(w=lib.Weights(t.values, badt, t.scales, t.global_scale,
                                              lib.LAYOUT_PAIRED_TILED))
    assert counts["masks"] == 1


def test_paired_canonical_rejected_by_gemm(lib):
    w = lib.pack_weights(torch.zeros(2, 32, 64, device="cuda"), paired=True)
    off = torch.tensor([0, 1, 1], dtype=torch.int32, device="cuda")
    x = torch.zeros(1, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.MoesqError) as ei:
        lib.grouped_spgemm(x, off, w)
    assert ei.value.status == lib.ERR_LAYOUT


# ------------------------------------------------------------------ grouped GEMM

def _paired_case(lib, loads, N, K, swiglu, seed):
    E = len(loads)
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    rng = np.random.default_rng(seed)
    ids = ids[rng.permutation(len(ids))]
    M = len(ids)
    wl = synth.Workload("edge", E=E, T=M, k=1, proj=(("w", N, K),), outliers=True,
                        bias="none", seed=seed)
    x = synth.tokens(wl, T=M, K=K)
    dense = synth.dense_experts(wl, 0)
    packs = [oracle.quantize_paired(dense[e].numpy()) for e in range(E)]
    w = lib.tile_weights(lib.pack_weights(dense.cuda(), paired=True))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, 1)
    xr = lib.permute(x.cuda(), perm, 1)
    y = lib.grouped_spgemm(xr, off, w, lib.EPI_SWIGLU if swiglu else lib.EPI_NONE)
    torch.cuda.synchronize()
    off_r, perm_r, _ = oracle.route(ids, E)
    dec = [oracle.decode_paired(p) for p in packs]
    y_ref = oracle.grouped_gemm(oracle.permute(x.to(torch.float64).numpy(), perm_r, 1), off_r,
                                lambda e: dec[e])
    if swiglu:
        y_ref = oracle.bf16_round(oracle.swiglu(y_ref))
    tol_check(f64(y), y_ref, f"paired loads={loads} N={N} K={K} swiglu={swiglu}")


@pytest.mark.parametrize("loads,N,K,swiglu", [
    ([0, 1, 15, 16, 17, 33, 130, 0], 64, 128, False),      # 16-row tile
    ([0, 1, 15, 16, 17, 33, 130, 0], 128, 192, True),      # 16-row tile, K tail, SwiGLU
    ([1] * 20, 128, 256, True),
    ([0, 0, 0, 200, 0], 288, 320, False),                  # 32-row tile, K tail
    ([5, 0, 64, 127, 128, 129, 1], 32, 448, False),        # 32-row tile, ragged tiles
    ([40] * 4, 64, 64, False),                             # K below one chunk
    ([300, 260], 576, 512, True),                          # 32-row tile, SwiGLU
    ([0, 3, 0, 1], 32, 64, False),
    # tile choice of a short call (one launch): M = 4E the one-fragment
    # streaming tile (an expert of 20 rows takes two token tiles); up to 32
    # rows per expert on average the two-fragment streaming tile, above it
    # the contraction tile
    ([20, 0, 10, 2, 0, 0, 0, 0], 64, 512, True),
    ([20, 1, 10, 2, 0, 0, 0, 0], 64, 512, False),
    ([80, 0, 40, 8], 128, 512, True),
    ([80, 1, 40, 8], 128, 512, False),
    # the largest expert count: 1024 experts of 0-2 rows
    ([(i * 7) % 3 for i in range(1024)], 32, 64, False),
])
def test_paired_spgemm_edges(lib, loads, N, K, swiglu):
    _paired_case(lib, loads, N, K, swiglu, seed=sum(loads) + N + K + 7)


def test_paired_tiny_end_to_end(lib):
    """tiny with paired weights: route -> permute -> GEMM -> weighted
    combine against the oracle."""
    wl = synth.WORKLOADS["tiny"]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    dense = synth.dense_experts(wl, 0)
    packs = [oracle.quantize_paired(dense[e].numpy()) for e in range(wl.E)]
    w = lib.tile_weights(lib.pack_weights(dense.cuda(), paired=True))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    y = lib.grouped_spgemm_gather(x.cuda(), perm, wl.k, off, w)
    out = lib.unpermute(y, inv, torch.from_numpy(tw).cuda(), wl.T, wl.k)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    dec = [oracle.decode_paired(p) for p in packs]
    y_ref = oracle.grouped_gemm(oracle.permute(x.to(torch.float64).numpy(), perm_r, wl.k), off_r,
                                lambda e: dec[e])
    tol_check(f64(y), y_ref, "Y")
    tol_check(f64(out), oracle.unpermute(y_ref, inv_r, tw, wl.T, wl.k), "weighted combine")


@pytest.mark.parametrize("name,swiglu", [("decode-30b", False), ("prefill-30b", False),
                                         ("decode-1t", True)])
def test_paired_gather_matches_permute(lib, name, swiglu):
    """Fused dispatch gives the bytes of permute + GEMM on paired weights,
    with out-of-range permutation entries giving zero rows."""
    wl = synth.WORKLOADS[name]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=True))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    x = synth.tokens(wl).cuda()
    epi = lib.EPI_SWIGLU if swiglu else lib.EPI_NONE
    bad = perm.clone()
    bad[[0, wl.M - 1]] = torch.tensor([-1, wl.M], dtype=torch.int32, device=bad.device)
    for p in (perm, bad):
        want = lib.grouped_spgemm(lib.permute(x, p, wl.k), off, w, epi)
        got = lib.grouped_spgemm_gather(x, p, wl.k, off, w, epi)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
    assert not got[[0, wl.M - 1]].any()


@pytest.mark.parametrize("name", ["decode-30b", "prefill-30b", "decode-1t", "prefill-1t"])
def test_paired_workloads(lib, name):
    """Full-size workloads with paired weights: gate/up (SwiGLU on the
    trillion-class chain) and, for the chain, the down projection.  Sampled
    experts (the largest, one from each launch range of row counts, a random
    one) against the oracle: packed bytes and every routed row."""
    wl = synth.WORKLOADS[name]
    ids, _ = synth.routing(wl)
    x = synth.tokens(wl)
    say(f"[{name}] packing paired experts on the GPU")
    w1 = pack_workload(lib, wl, 0, paired=True)
    w1t = lib.tile_weights(w1)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    epi = lib.EPI_SWIGLU if wl.swiglu else lib.EPI_NONE
    y1 = lib.grouped_spgemm_gather(x.cuda(), perm, wl.k, off, w1t, epi)
    y2 = None
    w2 = None
    if len(wl.proj) > 1:
        w2 = pack_workload(lib, wl, 1, paired=True)
        y2 = lib.grouped_spgemm(y1, off, lib.tile_weights(w2))
    torch.cuda.synchronize()
    off_r, perm_r, _ = oracle.route(ids, wl.E)
    counts = np.diff(off_r)
    x64 = x.to(torch.float64).numpy()
    rng = np.random.default_rng(wl.seed + 5)
    picks = pick_experts(counts, rng)
    say(f"[{name}] oracle for experts {picks} (rows {[int(counts[e]) for e in picks]})")
    ref1 = oracle_experts(wl, 0, picks, paired=True)
    ref2 = oracle_experts(wl, 1, picks, paired=True) if y2 is not None else None
    for e in picks:
        assert_same_pack(w1, e, ref1[e][0], f"{name} expert {e}")
        rows = np.arange(off_r[e], off_r[e + 1])
        ref = oracle.expert_gemm(x64[perm_r[rows] // wl.k], ref1[e][1])
        if wl.swiglu:
            ref = oracle.bf16_round(oracle.swiglu(ref))
        sel = torch.from_numpy(rows).cuda()
        tol_check(f64(y1[sel]), ref, f"{name} expert {e} ({counts[e]} rows)")
        if y2 is not None:
            assert_same_pack(w2, e, ref2[e][0], f"{name} down expert {e}")
            # the down GEMM from the oracle's own h, as the chain defines it
            tol_check(f64(y2[sel]), oracle.expert_gemm(ref, ref2[e][1]), f"{name} down expert {e}")
        say(f"[{name}] expert {e}: {counts[e]} rows ok")
