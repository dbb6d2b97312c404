"""Throughput of the grouped 4:8 sparse-FP4 expert path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic,
device-resident input:
  route -> permute -> grouped GEMM (gate/up, SwiGLU epilogue) -> grouped GEMM
  (down) -> router-weighted combine            (trillion-class workloads)
  route -> permute -> grouped GEMM -> combine  (30B-class workloads)
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
workload.
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
ROTATE_BYTES = 1 << 30        # weight replicas rotate until they span 1 GiB


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill-1t", choices=list(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain gather copy of known size (moesq_unpermute without "
                         "weights over 512 MiB in, 512 MiB out) to scale HBM byte counters")
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


def pack_on_gpu(m, wl, proj, chunk=16):
    """Dense weights drawn on the GPU, packed (canonical) and re-laid in the
    tiled layout the GEMM streams best."""
    _, N, K = wl.proj[proj]
    w = m.Weights.empty(wl.E, N, K)
    for c0 in range(0, wl.E, chunk):
        c1 = min(wl.E, c0 + chunk)
        dense = synth.dense_experts(wl, proj, range(c0, c1), device="cuda")
        m.moesq_pack_weights(dense, c1 - c0, N, K, w.values[c0:c1], w.masks[c0:c1],
                             w.scales[c0:c1], w.global_scale[c0:c1])
        del dense
    t = m.tile_weights(w)
    torch.cuda.synchronize()
    del w
    return t


class Step:
    """Buffers and launches of one pass of the hot path."""

    def __init__(self, m, wl):
        self.m, self.wl = m, wl
        dev = torch.device("cuda")
        ids, tw = synth.routing(wl)
        self.ids_host = ids
        self.ids = torch.from_numpy(ids).to(dev)
        self.tw = torch.from_numpy(tw).to(dev)
        self.x = synth.tokens(wl).to(dev)
        self.w = [pack_on_gpu(m, wl, p) for p in range(len(wl.proj))]
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
        self.xr = torch.empty(M, wl.K_in, **bf)
        if wl.swiglu:
            self.h = torch.empty(M, wl.proj[0][1] // 2, **bf)
            self.y = torch.empty(M, wl.proj[1][1], **bf)
        else:
            self.y = torch.empty(M, wl.proj[0][1], **bf)
        self.out = torch.empty(T if wl.weighted_combine else M, self.y.shape[1], **bf)
        self.names = ["route", "permute"] + [f"gemm_{p[0]}" for p in wl.proj] + ["combine"]

    def calls(self):
        """(name, launch) of every kernel of one step, on the next weight
        replica."""
        m, wl = self.m, self.wl
        w = self.replicas[self.turn % len(self.replicas)]
        self.turn += 1
        calls = [
            lambda: m.moesq_route(self.ids, wl.T, wl.k, wl.E, self.off, self.perm, self.inv,
                                  self.route_ws),
            lambda: m.moesq_permute(self.x, self.perm, wl.T, wl.k, wl.K_in, self.xr),
        ]
        if wl.swiglu:
            calls.append(lambda: m.moesq_grouped_spgemm(self.xr, self.off, wl.M, w[0],
                                                        m.EPI_SWIGLU, self.h))
            calls.append(lambda: m.moesq_grouped_spgemm(self.h, self.off, wl.M, w[1],
                                                        m.EPI_NONE, self.y))
        else:
            calls.append(lambda: m.moesq_grouped_spgemm(self.xr, self.off, wl.M, w[0],
                                                        m.EPI_NONE, self.y))
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


def measured_traffic(workload, proj_name):
    """HBM bytes per launch of the grouped GEMM from the committed rocprofv3
    counter summary, or None when the GEMM source has changed since the
    counters were taken (or no summary covers this workload)."""
    path = os.path.join(ROOT, "profiles", "spgemm_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    csrc = os.path.join(ROOT, "sparse_fp4_expert_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, n), "rb").read() for n in ("spgemm.hip", "common.hpp"))
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    k = rec.get("kernels", {}).get(f"{workload}/{proj_name}")
    return None if k is None else k.get("traffic_bytes")


def gemm_work(wl, ids):
    """Dense-equivalent flops and compressed weight bytes of the active
    experts, per projection."""
    counts = np.bincount(ids, minlength=wl.E)
    active = int((counts > 0).sum())
    res = []
    for _, N, K in wl.proj:
        flops = 2.0 * wl.M * N * K
        wbytes = active * (N * K * 13 // 32 + 4)
        res.append((flops, wbytes))
    return res, active


def cpu_baseline(wl, budget_s):
    """The CPU oracle on a bounded sample of the same workload: the experts
    with the most routed rows, each through oracle compression-decode and the
    float64 GEMM of all its rows (every projection), until the budget is
    spent.  Reported in the step's unit, scaled by the sampled share."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    ids, _ = synth.routing(wl)
    x = synth.tokens(wl).to(torch.float64).numpy()
    off, perm, _ = oracle.route(ids, wl.E)
    counts = np.diff(off)
    order = np.argsort(-counts, kind="stable")
    t0 = time.perf_counter()
    flops = 0.0
    wbytes = 0
    rows_done = 0
    experts = 0
    for e in order:
        if counts[e] == 0 or time.perf_counter() - t0 > budget_s:
            break
        rows = perm[off[e]:off[e + 1]] // wl.k
        a = x[rows]
        for p, (_, N, K) in enumerate(wl.proj):
            dense = synth.dense_expert(wl, p, int(e)).numpy()
            pk = oracle.quantize(dense)
            Wd = oracle.decode(pk)
            y = oracle.expert_gemm(a, Wd)
            if wl.swiglu and p == 0:
                a = oracle.bf16_round(oracle.swiglu(y))
            flops += 2.0 * len(rows) * N * K
            wbytes += pk.nbytes
        rows_done += len(rows)
        experts += 1
    dt = time.perf_counter() - t0
    sample = (f"{experts} experts with the most rows ({rows_done} of {wl.M} routed rows), "
              f"each: compress + decode + float64 GEMM of every projection")
    return flops, wbytes, dt, threads, sample


def main():
    args = parse()
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
    step = Step(m, wl)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    # Each step replays a HIP graph of its five or six launches, so that
    # short decode kernels are not separated by host launch gaps.
    graphs = step.capture_steps()
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    # Timed region: exactly `steps` steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    kernel_ms = step.kernel_ms(reps=max(8, len(step.replicas)))

    work, active = gemm_work(wl, step.ids_host)
    total_flops = sum(f for f, _ in work)
    total_wbytes = sum(b for _, b in work)
    prefill = wl.M >= 4096
    if prefill:
        value, unit = total_flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = total_wbytes / (ms_step * 1e-3) / 1e9, "GB/s"
    g0 = step.names[2]
    g0_ms = kernel_ms[g0]
    f0, b0 = work[0]
    if prefill:
        roof = {"bound": "mfma", "achieved": f0 / (g0_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b0 / (g0_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name, wl.proj[0][0])
    roof["kernel"] = f"moesq_grouped_spgemm ({wl.proj[0][0]})"
    roof["kernel_ms"] = g0_ms

    res = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "E": wl.E, "T": wl.T, "k": wl.k, "routed_rows": wl.M,
                      "projections": [list(p) for p in wl.proj], "routing": wl.bias,
                      "active_experts": active, "parallelism": "none"},
           "kernel_ms": kernel_ms,
           "weight_replicas": len(step.replicas),
           "gemm_tflops_dense_equiv": total_flops / 1e12,
           "weight_gb_active": total_wbytes / 1e9,
           "roofline": roof}
    if not args.no_cpu_baseline:
        fl, wb, dt, threads, sample = cpu_baseline(wl, args.cpu_seconds)
        cv = fl / dt / 1e12 if prefill else wb / dt / 1e9
        res["cpu_baseline"] = {"value": cv, "unit": unit, "cores": threads, "kind": "oracle",
                               "sample": sample, "seconds": dt}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
