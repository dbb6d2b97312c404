"""Host-side logic of bench.py (no GPU): the one-GPU guard, the work and
byte counts behind `value` and `roofline.achieved`, the traffic lookup, and
the CPU-baseline leg on the small workload."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "one process drives one GPU" in r.stderr


def test_expert_bytes_formats():
    # 4:8: 4 bits per kept value (half the positions) + 1 mask bit per
    # position + one E4M3 byte per 32 positions = 13/32 byte; paired: 11/32
    N, K = 4096, 7168
    assert bench.expert_bytes(N, K, False) == N * K // 2 // 2 + N * K // 8 + N * K // 32 + 4
    assert bench.expert_bytes(N, K, True) == N * K // 4 + N * K // 16 + N * K // 32 + 4


def test_gemm_work_counts_active_experts():
    for name in ("tiny", "decode-30b", "decode-1t"):
        wl = synth.WORKLOADS[name]
        ids, _ = synth.routing(wl)
        work, active = bench.gemm_work(wl, ids)
        assert active == len(np.unique(ids))
        for (flops, wbytes), (_, N, K) in zip(work, wl.proj):
            assert flops == 2.0 * wl.M * N * K
            assert wbytes == active * bench.expert_bytes(N, K, False)


def test_traffic_lookup_needs_a_known_workload():
    assert bench.measured_traffic("no-such-workload", "gate_up") is None
    v = bench.measured_traffic("prefill-1t", "gate_up")
    assert v is None or v > 0


import pytest  # noqa: E402


@pytest.mark.parametrize("paired", [False, True])
def test_cpu_baseline_tiny(paired):
    wl = synth.WORKLOADS["tiny"]
    work, dt, threads, sample, phases = bench.cpu_baseline(wl, 1.0, paired)
    assert dt > 0 and threads >= 1 and work > 0
    assert set(phases) >= {"route", "permute", "decode", "gemm", "combine"}
    assert "routed rows" in sample
