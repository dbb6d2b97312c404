"""W4A4 (NVFP4 activations, 32-position E4M3 blocks, one fp32 scale per row)
on the GPU against the oracle, through the C ABI: the quantizer bit-exact
(codes, scales, row scales) on hand-derived rows, edge rows and the workload
tokens; the W4A4 grouped GEMM within the tolerance of the bf16 outputs
against the oracle's float64 product of the dequantized activations and
weights, on edge loads for both weight formats and layouts, on the
three-launch path of large calls, at full size on the tiny and 30B-class
workloads (every element) and on sampled experts of the trillion-class
chain (quantized tokens gathered into gate/up with SwiGLU, the bf16 h
quantized again for down, the weighted combine)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pins
import synth
from gpu_util import (assert_same_pack, f64, oracle_decode, oracle_expert, oracle_experts,
                      pack_workload, pick_experts, tol_check)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _same_quant(q, ref, what):
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), ref.codes), f"{what}: codes differ"
    assert np.array_equal(q.scales.cpu().numpy(), ref.scales), f"{what}: scales differ"
    assert np.array_equal(q.row_scale.cpu().numpy(), ref.g), f"{what}: row scales differ"


def test_quantize_fixture(lib):
    d = {ln[0]: ln[1:] for ln in pins._lines("act_rows.txt")}
    x = torch.tensor([[float(v) for v in d["x0"]], [float(v) for v in d["x1"]]],
                     dtype=torch.float32).to(torch.bfloat16)
    q = lib.quantize_activations(x.cuda())
    torch.cuda.synchronize()
    for r in range(2):
        assert q.codes[r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"codes{r}"]]
        assert q.scales[r].cpu().numpy().tolist() == [int(t, 16) for t in d[f"scales{r}"]]
    assert q.row_scale.cpu().numpy().tolist() == [float(v) for v in d["g"]]


@pytest.mark.parametrize("T,K,seed", [(24, 256, 1), (37, 7168, 2), (8, 32, 3), (130, 2048, 4),
                                        (9, 8192, 5), (7, 8224, 6), (11, 4128, 7)])
def test_quantize_edge_rows(lib, T, K, seed):
    """Rows spanning 2^-17 to 2^17 in range, outlier channels, a zero row, a
    zero block, rows of ties and a negative row maximum; rows whose blocks
    do not fill the wave's lanes evenly, up to K = 8224."""
    x = pins._act_rows(np.random.default_rng(seed), T=T, K=K)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    q = lib.quantize_activations(xb.cuda())
    _same_quant(q, oracle.quantize_activations(xb.float().numpy()), f"T={T} K={K}")


@pytest.mark.parametrize("name", ["tiny", "decode-1t", "prefill-30b", "prefill-1t"])
def test_quantize_workload_tokens(lib, name):
    wl = synth.WORKLOADS[name]
    x = synth.tokens(wl)
    q = lib.quantize_activations(x.cuda())
    _same_quant(q, oracle.quantize_activations(x.float().numpy()), name)


def _w4a4_case(lib, loads, N, K, swiglu, paired, tiled, seed, flat=False):
    E = len(loads)
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    ids = ids[np.random.default_rng(seed).permutation(len(ids))]
    M = len(ids)
    wl = synth.Workload("w4a4-edge", E=E, T=M, k=1, proj=(("w", N, K),), outliers=True,
                        bias="none", seed=seed)
    x = synth.tokens(wl, T=M, K=K)
    w = pack_workload(lib, wl, 0, paired=paired)
    if tiled:
        w = lib.tile_weights(w)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, 1)
    xq = lib.quantize_activations(x.cuda())
    epi = (lib.EPI_SWIGLU if swiglu else lib.EPI_NONE) | (lib.OUT_FLAT if flat else 0)
    y = lib.grouped_spgemm_act4(xq, off, w, epi, perm=perm, k=1)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r = oracle.route(ids, E)
    dec = {e: oracle_decode(oracle_expert(wl, 0, e, paired=paired)) for e in range(E) if loads[e]}
    xt = oracle.decode_activations(oracle.quantize_activations(x.float().numpy()))
    y_ref = oracle.grouped_gemm(oracle.permute(xt, perm_r, 1), off_r, lambda e: dec[int(e)])
    if swiglu:
        y_ref = oracle.bf16_round(oracle.swiglu(y_ref))
    if flat:
        y_ref = oracle.unpermute(y_ref, inv_r, None, M, 1)
    tol_check(f64(y), y_ref, f"W4A4 loads={loads} N={N} K={K} swiglu={swiglu} paired={paired} "
                             f"tiled={tiled} flat={flat}")


@pytest.mark.parametrize("paired,tiled", [(False, False), (False, True), (True, True)],
                         ids=["4:8-canonical", "4:8-tiled", "paired"])
@pytest.mark.parametrize("loads,N,K,swiglu", [
    ([0, 1, 15, 16, 17, 33, 130, 0], 64, 128, False),      # streaming tiles, ragged tiles
    ([0, 1, 15, 16, 17, 33, 130, 0], 128, 192, True),      # K tail, SwiGLU
    ([1] * 20, 128, 256, True),                            # decode batch: one-fragment tile
    ([0, 0, 0, 200, 0], 288, 320, False),                  # contraction tile, K tail
    ([5, 0, 64, 127, 128, 129, 1], 32, 448, False),        # contraction tile, ragged tiles
    ([40] * 4, 64, 64, False),                             # K below one chunk
    ([300, 260], 576, 512, True),                          # contraction tile, SwiGLU
])
def test_w4a4_edges(lib, loads, N, K, swiglu, paired, tiled):
    _w4a4_case(lib, loads, N, K, swiglu, paired, tiled, seed=sum(loads) + N + K + 11)


def test_w4a4_flat_output(lib):
    _w4a4_case(lib, [0, 3, 17, 40, 1], 128, 256, False, False, True, seed=5, flat=True)
    _w4a4_case(lib, [0, 3, 17, 40, 1], 128, 256, False, True, True, seed=6, flat=True)


@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
def test_w4a4_split_launches(lib, paired):
    """A call of at least 5.5e11 multiply-adds: three launches over the
    experts of up to 16, 17-32 and more rows; all rows of the small experts
    and 256 of the large one against the oracle."""
    loads = [9, 16, 17, 25, 32, 33, 65468]
    N, K = 2048, 4096
    M = sum(loads)
    E = len(loads)
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    ids = ids[np.random.default_rng(78).permutation(M)]
    wl = synth.Workload("split", E=E, T=M, k=1, proj=(("w", N, K),), outliers=True,
                        bias="none", seed=4243)
    x = synth.tokens(wl, T=M, K=K)
    say(f"[W4A4 split launches] paired={paired}")
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), E, 1)
    xq = lib.quantize_activations(x.cuda())
    y = lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE, perm=perm, k=1)
    torch.cuda.synchronize()
    off_r, perm_r, _ = oracle.route(ids, E)
    ref = oracle_experts(wl, 0, range(E), paired=paired)
    xf = x.float().numpy()
    for e in range(E):
        rows = np.arange(off_r[e], off_r[e + 1])
        if len(rows) > 256:
            rows = np.concatenate([rows[:128], rows[-128:]])
        want = oracle.w4a4_expert_gemm(xf[perm_r[rows]], ref[e][1])
        tol_check(f64(y[torch.from_numpy(rows).cuda()]), want,
                  f"W4A4 split launches paired={paired} expert {e} ({loads[e]} rows)")


@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
@pytest.mark.parametrize("name", ["tiny", "decode-30b", "prefill-30b"])
def test_w4a4_full_tensor(lib, name, paired):
    """Every output element of the tiny and 30B-class workloads: quantized
    tokens gathered into the GEMM with the flat-order epilogue (the benchmark's
    W4A4 step), and in routed order followed by the weighted combine."""
    wl = synth.WORKLOADS[name]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    say(f"[{name}] W4A4 paired={paired}: packing")
    wc = pack_workload(lib, wl, 0, paired=paired)
    w = lib.tile_weights(wc)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    xq = lib.quantize_activations(x.cuda())
    flat = lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE | lib.OUT_FLAT, perm=perm, k=wl.k)
    y = lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE, perm=perm, k=wl.k)
    out = lib.unpermute(y, inv, torch.from_numpy(tw).cuda(), wl.T, wl.k)
    torch.cuda.synchronize()
    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    xqr = oracle.quantize_activations(x.float().numpy())
    _same_quant(xq, xqr, f"{name} tokens")
    active = np.nonzero(np.diff(off_r))[0]
    ref = oracle_experts(wl, 0, active, paired=paired)
    for e in active:
        assert_same_pack(wc, int(e), ref[int(e)][0], f"{name} expert {e}")
    xt = oracle.decode_activations(xqr)
    y_ref = oracle.grouped_gemm(oracle.permute(xt, perm_r, wl.k), off_r, lambda e: ref[int(e)][1])
    rel, mx = tol_check(f64(y), y_ref, f"{name} W4A4 Y")
    say(f"[{name}] W4A4 Y: rel Frobenius {rel:.2e}, max abs {mx:.2e}")
    tol_check(f64(flat), oracle.unpermute(y_ref, inv_r, None, wl.T, wl.k), f"{name} W4A4 flat Y")
    tol_check(f64(out), oracle.unpermute(y_ref, inv_r, tw, wl.T, wl.k), f"{name} W4A4 combine")


@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
@pytest.mark.parametrize("name", ["decode-1t", "prefill-1t"])
def test_w4a4_chain_1t(lib, name, paired):
    """The trillion-class W4A4 chain as the benchmark runs it: quantized
    tokens gathered into gate/up with SwiGLU, the bf16 h quantized per routed
    row (bit-exact against the oracle's quantization of the same h), down on
    the quantized h, weighted combine.  Sampled experts (the largest and one
    from each launch range) against the oracle chain: h from the oracle's
    W4A4 gate/up, Y2 from the oracle's quantization of its own h."""
    wl = synth.WORKLOADS[name]
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl)
    say(f"[{name}] W4A4 chain paired={paired}: packing")
    w1c = pack_workload(lib, wl, 0, paired=paired)
    w2c = pack_workload(lib, wl, 1, paired=paired)
    w1, w2 = lib.tile_weights(w1c), lib.tile_weights(w2c)
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    xq = lib.quantize_activations(x.cuda())
    h = lib.grouped_spgemm_act4(xq, off, w1, lib.EPI_SWIGLU, perm=perm, k=wl.k)
    hq = lib.quantize_activations(h)
    y2 = lib.grouped_spgemm_act4(hq, off, w2, lib.EPI_NONE)
    tw_d = torch.from_numpy(tw).cuda()
    out = lib.unpermute(y2, inv, tw_d if wl.weighted_combine else None, wl.T, wl.k)
    torch.cuda.synchronize()
    _same_quant(hq, oracle.quantize_activations(h.float().cpu().numpy()), f"{name} h")
    off_r, perm_r, inv_r = oracle.route(ids, wl.E)
    counts = np.diff(off_r)
    picks = pick_experts(counts, np.random.default_rng(wl.seed + 9), n_random=0)
    say(f"[{name}] oracle for experts {picks} (rows {[int(counts[e]) for e in picks]})")
    ref1 = oracle_experts(wl, 0, picks, paired=paired)
    ref2 = oracle_experts(wl, 1, picks, paired=paired)
    xf = x.float().numpy()
    for e in picks:
        assert_same_pack(w1c, e, ref1[e][0], f"{name} gate_up expert {e}")
        rows = np.arange(off_r[e], off_r[e + 1])
        y1_ref = oracle.w4a4_expert_gemm(xf[perm_r[rows] // wl.k], ref1[e][1])
        h_ref = oracle.bf16_round(oracle.swiglu(y1_ref))
        y2_ref = oracle.w4a4_expert_gemm(h_ref, ref2[e][1])
        sel = torch.from_numpy(rows).cuda()
        tol_check(f64(h[sel]), h_ref, f"{name} W4A4 h, expert {e}")
        tol_check(f64(y2[sel]), y2_ref, f"{name} W4A4 Y2, expert {e}")
        say(f"[{name}] expert {e}: {counts[e]} rows ok")
    want = oracle.unpermute(f64(y2), inv_r, tw if wl.weighted_combine else None, wl.T, wl.k)
    if wl.weighted_combine:
        tol_check(f64(out), want, f"{name} W4A4 weighted combine")
    else:
        assert np.array_equal(f64(out), want)


@pytest.mark.parametrize("paired", [False, True], ids=["4:8", "paired"])
def test_w4a4_gather_invalid_perm_entries(lib, paired):
    """Out-of-range permutation entries give zero rows (plain order) or no
    store at all (flat order), as with bf16 activations; the other rows are
    unchanged."""
    wl = synth.WORKLOADS["decode-30b"]
    ids, _ = synth.routing(wl)
    w = lib.tile_weights(pack_workload(lib, wl, 0, paired=paired))
    x = synth.tokens(wl).cuda()
    off, perm, inv = lib.route(torch.from_numpy(ids).cuda(), wl.E, wl.k)
    xq = lib.quantize_activations(x)
    want = lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE, perm=perm, k=wl.k)
    bad = perm.clone()
    lost = [0, wl.M // 2, wl.M - 1]
    bad[lost] = torch.tensor([-1, wl.M, 1 << 30], dtype=torch.int32, device=bad.device)
    got = lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE, perm=bad, k=wl.k)
    flat = torch.full_like(want, 7)
    lib.grouped_spgemm_act4(xq, off, w, lib.EPI_NONE | lib.OUT_FLAT, perm=bad, k=wl.k, out=flat)
    torch.cuda.synchronize()
    assert not got[lost].any()
    keep = torch.ones(wl.M, dtype=torch.bool, device=got.device)
    keep[lost] = False
    assert torch.equal(got[keep], want[keep])
    gone = perm[lost].long()                       # flat rows nobody writes now
    fkeep = torch.ones(wl.M, dtype=torch.bool, device=got.device)
    fkeep[gone] = False
    assert bool((flat[~fkeep] == 7).all())
    assert torch.equal(flat[perm[keep].long()], want[keep])
