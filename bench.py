"""Throughput of the grouped 4:8 sparse-FP4 expert path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--sweep] [--paired]

One step is one pass of the whole hot path over one batch of synthetic,
device-resident input:
  route -> dispatch + grouped GEMM (gate/up, SwiGLU epilogue) -> grouped GEMM
  (down) -> router-weighted combine            (trillion-class workloads)
  route -> dispatch + grouped GEMM -> scatter to flat order  (30B-class workloads)
The dispatch (gather of the routed token rows) runs inside the first GEMM,
and for decode batches (T*k <= 1024 and <= 4E) the routing too
(moesq_route_grouped_spgemm); the 30B-class scatter (no router weights) is
the GEMM's epilogue storing each row at its flat position (MOESQ_OUT_FLAT).
--unfused runs route, permute and the scatter as kernels of their own.
Inputs (tokens, top-k ids, router weights, packed expert weights) are built
and packed on the GPU before timing.  Every step replays a HIP graph of its
launches; the timed region is bracketed by a device synchronisation on both
sides.  Per-kernel durations come from HIP events recorded on the launch
stream around a graph of back-to-back launches of that kernel alone, with
the weight replicas rotating as in the steps.

Prints one JSON line.  value = dense-equivalent GEMM TFLOP/s of the whole
step (2*M*N*K summed over the projections, divided by the step time) for
prefill workloads, compressed-weight GB/s of the active experts for decode
workloads.  `roofline` covers the dominant kernel (the first grouped GEMM);
`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.  Decode lines also carry the rate of a plain streaming read of
4 GiB on the same device (`read_ceiling_gbs`), the practical bound of a
weight stream.

--paired runs the same step on paired 4:8 weights (two of the four position
pairs of a group kept, 2.75 bits per weight) through the sparse MFMA.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "grouped sparse-FP4 GEMM TFLOP/s + weight GB/s (% of MFMA/HBM peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 MFMA
ROTATE_BYTES = 1 << 30        # weight replicas rotate until they span 1 GiB


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: enough for about 0.25 s of timed work, 20 to 4000)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill-1t", choices=list(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--unfused", action="store_true",
                    help="run the dispatch as its own permute kernel instead of inside the first GEMM")
    ap.add_argument("--separate-route", action="store_true",
                    help="decode batches: keep routing in its own kernel instead of the first GEMM")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of steps: time the first grouped GEMM of --workload over a grid "
                         "of active-expert counts G x rows per expert R (one JSON line per point)")
    ap.add_argument("--sweep-experts", default="1,4,16,64,128,384",
                    help="comma-separated active-expert counts G of --sweep")
    ap.add_argument("--sweep-rows", default="1,2,4,8,16,32,64",
                    help="comma-separated rows per expert R of --sweep")
    ap.add_argument("--paired", action="store_true",
                    help="paired 4:8 weights (2.75 bits per weight) on the sparse MFMA instead of "
                         "the unconstrained 4:8 format")
    ap.add_argument("--w4a4", action="store_true",
                    help="NVFP4 activations (W4A4): tokens quantized once per step, gathered as "
                         "FP4 rows into the first GEMM; the SwiGLU output quantized for the down GEMM")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain gather copy of known size (moesq_unpermute without "
                         "weights over 512 MiB in, 512 MiB out) to scale HBM byte counters")
    ap.add_argument("--record-counters", metavar="DIR",
                    help="no GPU: read the rocprofv3 counter CSVs under DIR (DIR/<case>/<pass>/..., "
                         "case = a workload name, <workload>_paired, or calibrate) and write "
                         "profiles/spgemm_counters.json")
    return ap.parse_args()


def calibrate_copy(m, reps=3):
    """A copy kernel of known traffic: every row of a [65536, 4096] bf16
    tensor is read once and written once (512 MiB each way)."""
    rows, n = 65536, 4096
    dev = torch.device("cuda")
    y = torch.ones(rows, n, dtype=torch.bfloat16, device=dev)
    inv = torch.randperm(rows, device=dev).to(torch.int32)
    out = torch.empty_like(y)
    for _ in range(reps):
        m.moesq_unpermute(y, inv, None, rows, 1, n, out)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "gather copy", "bytes_read_per_launch": rows * n * 2,
                      "bytes_written_per_launch": rows * n * 2, "launches": reps}))


def read_ceiling(m, nbytes=4 << 30, reps=10):
    """Practical HBM read ceiling: GB/s of the library's plain streaming-read
    kernel over a buffer far larger than the L2s and the MALL, timed with HIP
    events on the launch stream (best of `reps` launches after one warm-up)."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.moesq_stream_read(buf, sink)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        m.moesq_stream_read(buf, sink)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf
    return nbytes / (best * 1e-3) / 1e9


def expert_bytes(N, K, paired):
    """Compressed bytes of one expert: 13/32 byte per weight (4:8 masks) or
    11/32 (paired pattern indices), plus the fp32 global scale."""
    return N * K * (11 if paired else 13) // 32 + 4


def pack_on_gpu(m, wl, proj, chunk=16, paired=False):
    """Dense weights drawn on the GPU, packed (canonical, or canonical
    paired) and re-laid in the tiled layout the GEMM streams best."""
    _, N, K = wl.proj[proj]
    w = m.Weights.empty(wl.E, N, K, layout=m.LAYOUT_PAIRED if paired else m.LAYOUT_CANONICAL)
    pack = m.moesq_pack_weights_paired if paired else m.moesq_pack_weights
    for c0 in range(0, wl.E, chunk):
        c1 = min(wl.E, c0 + chunk)
        dense = synth.dense_experts(wl, proj, range(c0, c1), device="cuda")
        pack(dense, c1 - c0, N, K, w.values[c0:c1], w.masks[c0:c1], w.scales[c0:c1],
             w.global_scale[c0:c1])
        del dense
    t = m.tile_weights(w)
    torch.cuda.synchronize()
    del w
    return t


class Step:
    """Buffers and launches of one pass of the hot path."""

    def __init__(self, m, wl, fused=True, paired=False, separate_route=False, w4a4=False):
        self.m, self.wl, self.fused, self.w4a4 = m, wl, fused, w4a4
        dev = torch.device("cuda")
        ids, tw = synth.routing(wl)
        self.ids_host = ids
        self.ids = torch.from_numpy(ids).to(dev)
        self.tw = torch.from_numpy(tw).to(dev)
        self.x = synth.tokens(wl).to(dev)
        self.w = [pack_on_gpu(m, wl, p, paired=paired) for p in range(len(wl.proj))]
        # Weight sets smaller than ~1 GB would stay in the 256 MB Infinity
        # Cache across steps; rotate through replicas so that every step
        # streams its weights from HBM, as a serving step does.
        total = sum(w.nbytes for w in self.w)
        self.replicas = [self.w]
        for _ in range(max(0, -(-ROTATE_BYTES // total) - 1)):
            self.replicas.append([m.Weights(w.values.clone(), w.masks.clone(), w.scales.clone(),
                                            w.global_scale.clone(), w.layout) for w in self.w])
        self.turn = 0
        E, M, T, k = wl.E, wl.M, wl.T, wl.k
        i32 = dict(dtype=torch.int32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.off = torch.empty(E + 1, **i32)
        self.perm = torch.empty(M, **i32)
        self.inv = torch.empty(M, **i32)
        nws = m.moesq_route_workspace_bytes(T, k, E)
        self.route_ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        self.xr = None if fused else torch.empty(M, wl.K_in, **bf)
        if wl.swiglu:
            self.h = torch.empty(M, wl.proj[0][1] // 2, **bf)
            self.y = torch.empty(M, wl.proj[1][1], **bf)
        else:
            self.y = torch.empty(M, wl.proj[0][1], **bf)
        self.out = torch.empty(T if wl.weighted_combine else M, self.y.shape[1], **bf)
        # W4A4: the tokens' NVFP4 rows, and the SwiGLU output's for the down GEMM
        if w4a4:
            self.xq = m.Act4.empty(T, wl.K_in)
            self.hq = m.Act4.empty(M, wl.proj[0][1] // 2) if wl.swiglu else None
        # decode batches route inside the first GEMM's launch (bf16 activations)
        self.route_in_gemm = (fused and not separate_route and not w4a4 and M <= 1024
                              and M <= 4 * E)
        # without router weights the combine is a pure scatter to flat order:
        # with dispatch fused, the GEMM's epilogue stores there directly
        self.scatter_in_gemm = fused and not wl.weighted_combine and not wl.swiglu
        self.names = (([] if self.route_in_gemm else ["route"]) + ([] if fused else ["permute"])
                      + (["quantize_x"] if w4a4 else []) + [f"gemm_{wl.proj[0][0]}"]
                      + (["quantize_h"] if w4a4 and wl.swiglu else [])
                      + [f"gemm_{p[0]}" for p in wl.proj[1:]]
                      + ([] if self.scatter_in_gemm else ["combine"]))

    def calls(self):
        """(name, launch) of every kernel of one step, on the next weight
        replica."""
        m, wl = self.m, self.wl
        w = self.replicas[self.turn % len(self.replicas)]
        self.turn += 1
        calls = []
        if not self.route_in_gemm:
            calls.append(lambda: m.moesq_route(self.ids, wl.T, wl.k, wl.E, self.off, self.perm,
                                               self.inv, self.route_ws))
        if not self.fused:
            calls.append(lambda: m.moesq_permute(self.x, self.perm, wl.T, wl.k, wl.K_in, self.xr))

        if self.w4a4:
            calls.append(lambda: m.moesq_quantize_activations(self.x, wl.T, wl.K_in, self.xq.codes,
                                                              self.xq.scales, self.xq.row_scale))

        def first(epi, out):
            # routing and dispatch fused into the first GEMM, dispatch fused,
            # or the routed copy
            if self.w4a4:
                return lambda: m.moesq_grouped_spgemm_act4(self.xq, self.perm, wl.T, wl.k, self.off,
                                                           wl.M, w[0], epi, out)
            if self.route_in_gemm:
                return lambda: m.moesq_route_grouped_spgemm(self.ids, self.x, wl.T, wl.k, w[0], epi,
                                                            out, self.off, self.perm, self.inv)
            if self.fused:
                return lambda: m.moesq_grouped_spgemm_gather(self.x, self.perm, wl.T, wl.k, self.off,
                                                             w[0], epi, out)
            return lambda: m.moesq_grouped_spgemm(self.xr, self.off, wl.M, w[0], epi, out)

        if wl.swiglu:
            calls.append(first(m.EPI_SWIGLU, self.h))
            if self.w4a4:
                calls.append(lambda: m.moesq_quantize_activations(self.h, wl.M, self.h.shape[1],
                                                                  self.hq.codes, self.hq.scales,
                                                                  self.hq.row_scale))
                calls.append(lambda: m.moesq_grouped_spgemm_act4(self.hq, None, 0, 1, self.off, wl.M,
                                                                 w[1], m.EPI_NONE, self.y))
            else:
                calls.append(lambda: m.moesq_grouped_spgemm(self.h, self.off, wl.M, w[1],
                                                            m.EPI_NONE, self.y))
        elif self.scatter_in_gemm:
            calls.append(first(m.EPI_NONE | m.OUT_FLAT, self.out))
        else:
            calls.append(first(m.EPI_NONE, self.y))
        if not self.scatter_in_gemm:
            tw = self.tw if wl.weighted_combine else None
            calls.append(lambda: m.moesq_unpermute(self.y, self.inv, tw, wl.T, wl.k,
                                                   self.y.shape[1], self.out))
        return list(zip(self.names, calls))

    def run(self):
        for _, c in self.calls():
            c()

    def capture_steps(self):
        """One HIP graph of the whole step per weight replica (the graph
        holds that replica's weight pointers)."""
        graphs = []
        for _ in range(len(self.replicas)):
            g = torch.cuda.CUDAGraph()
            launches = self.calls()
            with torch.cuda.graph(g):
                for _, c in launches:
                    c()
            graphs.append(g)
        return graphs

    def kernel_ms(self, reps):
        """Average duration of each kernel of the step: HIP events on the
        launch stream around a graph of `reps` back-to-back launches of that
        kernel alone (weight replicas rotating), replayed twice."""
        res = {}
        n = len(self.names)
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            launches = [self.calls()[i][1] for _ in range(reps)]
            with torch.cuda.graph(g):
                for c in launches:
                    c()
            g.replay()
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev[0].record()
            g.replay()
            g.replay()
            ev[1].record()
            torch.cuda.synchronize()
            res[self.names[i]] = ev[0].elapsed_time(ev[1]) / (2 * reps)
            del g
        return res


def sweep(m, wl, Gs=(1, 4, 16, 64, 128, 384), Rs=(1, 2, 4, 8, 16, 32, 64), launches=16,
          paired=False):
    """Grouped GEMM of the workload's first projection (plain epilogue) over
    G active experts with R routed rows each, as the pages sweep expert-group
    count x rows per expert.  Each launch reads a different window of G
    experts (and weight replicas rotate when the whole set is under 1 GiB),
    so weights come from HBM; times are HIP events around a graph of
    `launches` back-to-back launches."""
    _, N, K = wl.proj[0]
    dev = torch.device("cuda")
    w0 = pack_on_gpu(m, wl, 0, paired=paired)
    reps = [w0] + [m.Weights(w0.values.clone(), w0.masks.clone(), w0.scales.clone(),
                             w0.global_scale.clone(), w0.layout)
                   for _ in range(max(0, -(-ROTATE_BYTES // w0.nbytes) - 1))]
    gen = torch.Generator(device="cpu").manual_seed(wl.seed + 77)
    for G in Gs:
        if G > wl.E:
            continue
        for R in Rs:
            M = G * R
            x = (torch.randn(M, K, generator=gen) * 1.0).to(torch.bfloat16).to(dev)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            offs = []
            for i in range(launches):
                start = (i // len(reps)) * G % wl.E
                counts = np.zeros(wl.E, np.int64)
                counts[(start + np.arange(G)) % wl.E] = R
                offs.append(torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev))
            calls = [(lambda o=offs[i], w=reps[i % len(reps)]:
                      m.moesq_grouped_spgemm(x, o, M, w, m.EPI_NONE, y)) for i in range(launches)]
            for c in calls[:2]:
                c()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in calls:
                    c()
            g.replay()
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev[0].record()
            g.replay()
            ev[1].record()
            torch.cuda.synchronize()
            us = 1e3 * ev[0].elapsed_time(ev[1]) / launches
            wbytes = G * expert_bytes(N, K, paired)
            print(json.dumps({"sweep": wl.name, "paired": paired, "N": N, "K": K, "G": G, "R": R,
                              "M": M,
                              "kernel_us": round(us, 2),
                              "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
                              "hbm_frac": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3),
                              "tflops_dense_eq": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1),
                              "weight_replicas": len(reps)}), flush=True)
            del g


COUNTERS_JSON = os.path.join(ROOT, "profiles", "spgemm_counters.json")
COPY_BYTES = 65536 * 4096 * 2          # calibrate_copy: bytes read and bytes written


def gemm_source_sha():
    """Hash of the GEMM's sources: counters taken on other sources are stale."""
    csrc = os.path.join(ROOT, "sparse_fp4_expert_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, n), "rb").read() for n in ("spgemm.hip", "common.hpp"))
    return hashlib.sha256(src).hexdigest()


def counter_key(workload, proj_name, paired=False, w4a4=False):
    return f"{workload}/{proj_name}" + ("/paired" if paired else "") + ("/w4a4" if w4a4 else "")


def measured_counters(workload, proj_name, paired=False, w4a4=False):
    """Per-call counter figures of the grouped GEMM from the committed
    rocprofv3 summary (traffic_bytes, mfma_flops, ...), or {} when the GEMM
    source has changed since the counters were taken (or no summary covers
    this workload)."""
    try:
        with open(COUNTERS_JSON) as f:
            rec = json.load(f)
    except OSError:
        return {}
    if gemm_source_sha() != rec.get("source_sha256"):
        return {}
    return rec.get("kernels", {}).get(counter_key(workload, proj_name, paired, w4a4), {})


def _kernel_tile(name):
    """(MS, SWIGLU) of a grouped-GEMM kernel from its demangled name, or None."""
    import re
    m = re.search(r"spgemm_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (true|false), (\d+)", name)
    if not m:
        return None
    return int(m.group(2)), m.group(6) == "true"


def record_counters(root):
    """Turns rocprofv3 counter CSVs into profiles/spgemm_counters.json.

    Layout: root/<case>/<pass>/.../*counter_collection.csv with case a
    workload name with the suffixes _paired and _w4a4 of the bench options
    it ran with, or calibrate (bench.py
    --calibrate-copy).  Per kernel: the mean over its dispatches of each
    counter; per GEMM call: the sum over the kernels of that projection (one
    to three launches).  HBM bytes = FETCH_SIZE and WRITE_SIZE (KiB) times
    the factor that makes the calibration copy read and write its known
    512 MiB; executed MFMA flops = SQ_INSTS_MFMA (wave instructions) times
    the multiply-adds of one instruction x 2 (32x32x16 and the sparse
    32x32x32: 32768; 16x16x32 and the sparse 16x16x64: 16384)."""
    import csv
    import glob
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))   # case -> kernel -> (dispatch, counter)
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        case = os.path.relpath(path, root).split(os.sep)[0]
        with open(path) as f:
            for row in csv.DictReader(f):
                key = (row.get("Dispatch_Id") or row.get("Correlation_Id"), row["Counter_Name"])
                per[case][row["Kernel_Name"]][key] += float(row["Counter_Value"])

    def means(kernel_rows):
        by = defaultdict(list)
        for (_, ctr), v in kernel_rows.items():
            by[ctr].append(v)
        return {c: sum(v) / len(v) for c, v in by.items()}

    cal = {}
    for name, rows in per.get("calibrate", {}).items():
        if "unpermute" in name:
            cal = means(rows)
    if "FETCH_SIZE" not in cal or "WRITE_SIZE" not in cal:
        raise SystemExit("record-counters: the calibrate case needs FETCH_SIZE and WRITE_SIZE of the copy")
    ff = COPY_BYTES / 1024 / cal["FETCH_SIZE"]
    wf = COPY_BYTES / 1024 / cal["WRITE_SIZE"]
    about = ("Per call of the grouped GEMM (the sum over the one to three launches of the "
             "call; each launch the mean over its dispatches): rocprofv3 counters; traffic_bytes "
             "= FETCH_SIZE and WRITE_SIZE (KiB) scaled so that a gather copy of known size "
             "(bench.py --calibrate-copy) reads and writes its 512 MiB; mfma_flops = "
             "SQ_INSTS_MFMA x 2 x the multiply-adds one MFMA instruction executes.")
    out = {"about": about,
           "calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_size_kib": cal["FETCH_SIZE"],
                           "fetch_factor": ff, "write_size_kib": cal["WRITE_SIZE"],
                           "write_factor": wf},
           "source_sha256": gemm_source_sha(), "kernels": {}}
    for case, kernels in sorted(per.items()):
        if case == "calibrate":
            continue
        name = case
        w4a4 = name.endswith("_w4a4")
        name = name[:-len("_w4a4")] if w4a4 else name
        paired = name.endswith("_paired")
        wl = synth.WORKLOADS[name[:-len("_paired")] if paired else name]
        for p, (pname, _, _) in enumerate(wl.proj):
            acc = defaultdict(float)
            names = []
            for name, rows in kernels.items():
                tile = _kernel_tile(name)
                if tile is None or (len(wl.proj) > 1 and tile[1] != (p == 0)):
                    continue
                names.append(name)
                m = means(rows)
                for c, v in m.items():
                    acc[c] += v
                if "SQ_INSTS_MFMA" in m:
                    acc["mfma_flops"] += m["SQ_INSTS_MFMA"] * (32768 if tile[0] == 32 else 16384)
            if not names:
                continue
            rec = {"launches": len(names), "kernels": sorted(names)}
            rec.update({c: round(v, 2) for c, v in acc.items()})
            if "FETCH_SIZE" in acc and "WRITE_SIZE" in acc:
                rec["traffic_bytes"] = acc["FETCH_SIZE"] * 1024 * ff + acc["WRITE_SIZE"] * 1024 * wf
            out["kernels"][counter_key(wl.name, pname, paired, w4a4)] = rec
    with open(COUNTERS_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {COUNTERS_JSON}: {sorted(out['kernels'])}")


def gemm_work(wl, ids, paired=False):
    """Dense-equivalent flops and compressed weight bytes of the active
    experts, per projection."""
    counts = np.bincount(ids, minlength=wl.E)
    active = int((counts > 0).sum())
    res = []
    for _, N, K in wl.proj:
        flops = 2.0 * wl.M * N * K
        wbytes = active * expert_bytes(N, K, paired)
        res.append((flops, wbytes))
    return res, active


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(wl, budget_s, paired=False, w4a4=False):
    """The CPU oracle on the same workload, each phase timed on its own.

    Route, permute and the combine run on the whole workload (data movement;
    the combine reads a zero Y of the right shape).  Decode, the float64 GEMM
    of every projection and SwiGLU run on the experts with the most routed
    rows until about `budget_s` seconds are spent, and are scaled to all
    active experts by their share of the GEMM flops (prefill) or of the
    compressed weight bytes (decode).  Compressing the dense weights (the
    packer, untimed on the GPU too) is timed but left out of the total.
    Returns (work, seconds, threads, sample, phases)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    ids, tw = synth.routing(wl)
    x = synth.tokens(wl).to(torch.float64).numpy()
    ph = dict.fromkeys(["route", "permute", "compress", "decode", "quantize", "gemm", "swiglu",
                        "combine"], 0.0)

    t = time.perf_counter()
    off, perm, inv = oracle.route(ids, wl.E)
    ph["route"] = time.perf_counter() - t
    t = time.perf_counter()
    oracle.permute(x, perm, wl.k)
    ph["permute"] = time.perf_counter() - t
    n_out = wl.proj[-1][1]
    y_zero = np.zeros((wl.M, n_out), np.float64)
    t = time.perf_counter()
    oracle.unpermute(y_zero, inv, tw if wl.weighted_combine else None, wl.T, wl.k)
    ph["combine"] = time.perf_counter() - t
    del y_zero

    counts = np.diff(off)
    active = int((counts > 0).sum())
    order = np.argsort(-counts, kind="stable")
    flops_all = sum(2.0 * wl.M * N * K for _, N, K in wl.proj)
    bytes_all = sum(active * expert_bytes(N, K, paired) for _, N, K in wl.proj)
    t0 = time.perf_counter()
    flops = 0.0
    wbytes = 0
    rows_done = experts = 0
    for e in order:
        if counts[e] == 0 or time.perf_counter() - t0 > budget_s:
            break
        rows = perm[off[e]:off[e + 1]] // wl.k
        a = x[rows]
        for p, (_, N, K) in enumerate(wl.proj):
            dense = synth.dense_expert(wl, p, int(e)).numpy()
            t = time.perf_counter()
            pk = oracle.quantize_paired(dense) if paired else oracle.quantize(dense)
            ph["compress"] += time.perf_counter() - t
            t = time.perf_counter()
            Wd = oracle.decode_paired(pk) if paired else oracle.decode(pk)
            ph["decode"] += time.perf_counter() - t
            if w4a4:
                t = time.perf_counter()
                a = oracle.decode_activations(oracle.quantize_activations(a))
                ph["quantize"] += time.perf_counter() - t
            t = time.perf_counter()
            y = oracle.expert_gemm(a, Wd)
            ph["gemm"] += time.perf_counter() - t
            if wl.swiglu and p == 0:
                t = time.perf_counter()
                a = oracle.bf16_round(oracle.swiglu(y))
                ph["swiglu"] += time.perf_counter() - t
            flops += 2.0 * len(rows) * N * K
            wbytes += pk.nbytes
        rows_done += len(rows)
        experts += 1
    prefill = wl.M >= 4096
    scale = flops_all / flops if prefill else bytes_all / wbytes
    total = ph["route"] + ph["permute"] + ph["combine"] + scale * (ph["decode"] + ph["quantize"]
                                                                  + ph["gemm"] + ph["swiglu"])
    sample = (f"route, permute and combine of all {wl.M} routed rows; decode"
              f"{' + NVFP4 activation quantization' if w4a4 else ''} + float64 GEMM"
              f"{' + SwiGLU' if wl.swiglu else ''} of the {experts} experts with the most rows "
              f"({rows_done} rows), scaled x{scale:.1f} to all {active} active experts")
    phases = {k: round(v, 4) for k, v in ph.items()}
    phases["scaled_to_all_experts"] = round(scale, 3)
    work = flops_all if prefill else bytes_all
    return work, total, threads, sample, phases


def main():
    args = parse()
    if args.record_counters:
        record_counters(args.record_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              "(one process drives one GPU; expert sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    from sparse_fp4_expert_amd import moesq as m
    if args.calibrate_copy:
        calibrate_copy(m)
        return
    wl = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(m, wl, Gs=tuple(int(v) for v in args.sweep_experts.split(",")),
              Rs=tuple(int(v) for v in args.sweep_rows.split(",")), paired=args.paired)
        return
    if args.w4a4 and args.unfused:
        sys.exit("--w4a4 gathers the quantized tokens inside the GEMM; --unfused does not apply")
    step = Step(m, wl, fused=not args.unfused, paired=args.paired,
                separate_route=args.separate_route, w4a4=args.w4a4)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    # Each step replays a HIP graph of its five or six launches, so that
    # short decode kernels are not separated by host launch gaps.
    graphs = step.capture_steps()
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    if args.steps is None:
        # short steps are timed over more replays, long ones over at least 20
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(len(graphs)):
            graphs[i].replay()
        torch.cuda.synchronize()
        est = (time.perf_counter() - t) / len(graphs)
        args.steps = int(min(4000, max(20, 0.25 / max(est, 1e-6))))
    # Timed region: exactly `steps` steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    kernel_ms = step.kernel_ms(reps=max(8, len(step.replicas)))

    work, active = gemm_work(wl, step.ids_host, args.paired)
    total_flops = sum(f for f, _ in work)
    total_wbytes = sum(b for _, b in work)
    prefill = wl.M >= 4096
    if prefill:
        value, unit = total_flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = total_wbytes / (ms_step * 1e-3) / 1e9, "GB/s"
    g0 = f"gemm_{wl.proj[0][0]}"
    g0_ms = kernel_ms[g0]
    f0, b0 = work[0]
    cnt = measured_counters(wl.name, wl.proj[0][0], args.paired, args.w4a4)
    if prefill:
        # The method's own work: one multiply-add per kept weight (half of the
        # N x K weights) per routed row, i.e. M*N*K flops per projection.
        roof = {"bound": "mfma", "achieved": 0.5 * f0 / (g0_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "work": "useful: M*N*K flops (one multiply-add per kept weight and routed row)"}
        roof["dense_equiv_tflops"] = f0 / (g0_ms * 1e-3) / 1e12
        # MFMA work the kernels execute, from the committed rocprofv3
        # SQ_INSTS_MFMA count of the same GEMM source (null when stale): it
        # includes the zeros of the 4:8 groups that the dense MFMA multiplies
        # and the padding of each expert's rows to whole fragments.
        mf = cnt.get("mfma_flops")
        roof["mfma_executed_tflops"] = None if mf is None else mf / (g0_ms * 1e-3) / 1e12
        roof["mfma_executed_frac"] = (None if mf is None
                                      else roof["mfma_executed_tflops"] / PEAK_BF16_TFLOPS)
        if args.w4a4:
            # NVFP4 operands with E4M3 block scales run on the bf16 MFMA after
            # an exact decode (the FP4 MFMA takes power-of-two block scales
            # only); the FP4 peak is shown for reference.
            roof["mfma_dtype"] = "bf16 (NVFP4 activations decoded exactly)"
            roof["fp4_peak"] = PEAK_FP4_TFLOPS
            roof["frac_of_fp4_peak"] = roof["achieved"] / PEAK_FP4_TFLOPS
    else:
        roof = {"bound": "hbm", "achieved": b0 / (g0_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
        # The published peak is the pin rate; a plain read stream on the
        # same device gives the rate a weight-streaming kernel can reach.
        ceil = read_ceiling(m)
        roof["read_ceiling_gbs"] = ceil
        roof["frac_of_read_ceiling"] = roof["achieved"] / ceil
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = cnt.get("traffic_bytes")
    roof["kernel"] = f"moesq_grouped_spgemm ({wl.proj[0][0]})"
    roof["kernel_ms"] = g0_ms

    res = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "E": wl.E, "T": wl.T, "k": wl.k, "routed_rows": wl.M,
                      "projections": [list(p) for p in wl.proj], "routing": wl.bias,
                      "active_experts": active, "parallelism": "none",
                      "weights": "paired 4:8 (2.75 bpw)" if args.paired else "4:8 (3.25 bpw)",
                      "activations": ("NVFP4 (E2M1, E4M3 per 32 positions, fp32 per row)"
                                      if args.w4a4 else "bf16")},
           "kernel_ms": kernel_ms,
           "weight_replicas": len(step.replicas),
           "gemm_tflops_dense_equiv": total_flops / 1e12,
           "weight_gb_active": total_wbytes / 1e9,
           "roofline": roof}
    if not args.no_cpu_baseline:
        work, dt, threads, sample, phases = cpu_baseline(wl, args.cpu_seconds, args.paired,
                                                         args.w4a4)
        cv = work / dt / 1e12 if prefill else work / dt / 1e9
        res["cpu_baseline"] = {"value": cv, "unit": unit, "cores": threads, "kind": "oracle",
                               "sample": sample, "seconds_full_step": dt, "phases_s": phases,
                               "cpu": cpu_model()}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
