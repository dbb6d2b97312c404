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


def test_counter_lookup_needs_a_known_workload():
    assert bench.measured_counters("no-such-workload", "gate_up") == {}
    v = bench.measured_counters("prefill-1t", "gate_up").get("traffic_bytes")
    assert v is None or v > 0


def test_record_counters_sums_launches_and_scales(tmp_path, monkeypatch):
    """Counter CSVs -> per-call figures: each kernel's mean over its
    dispatches, summed over the launches of one projection (the SwiGLU tiles
    are gate/up, the plain ones down); bytes scaled by the calibration copy;
    MFMA flops by the tile's instruction shape."""
    def csv(path, rows):
        path.parent.mkdir(parents=True, exist_ok=True)
        path.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n" +
                        "".join(f'{d},"{k}",{c},{v}\n' for d, k, c, v in rows))
    big = "void moesq::spgemm_kernel<8, 32, 2, 4, 128, true, 1, false>(moesq::SpgemmArgs)"
    small = "void moesq::spgemm_kernel<4, 16, 2, 1, 256, true, 1, false>(moesq::SpgemmArgs)"
    down = "void moesq::spgemm_kernel<8, 32, 2, 4, 128, false, 1, false>(moesq::SpgemmArgs)"
    copy = "void moesq::unpermute_kernel(args)"
    csv(tmp_path / "calibrate" / "f" / "run_counter_collection.csv",
        [(1, copy, "FETCH_SIZE", 262144), (2, copy, "FETCH_SIZE", 262144)])
    csv(tmp_path / "calibrate" / "w" / "run_counter_collection.csv", [(1, copy, "WRITE_SIZE", 524288)])
    csv(tmp_path / "prefill-1t" / "m" / "x" / "run_counter_collection.csv",
        [(5, big, "SQ_INSTS_MFMA", 1000), (6, big, "SQ_INSTS_MFMA", 3000),
         (7, small, "SQ_INSTS_MFMA", 100), (8, down, "SQ_INSTS_MFMA", 50),
         (5, big, "FETCH_SIZE", 10), (7, small, "FETCH_SIZE", 6), (5, big, "WRITE_SIZE", 4),
         (7, small, "WRITE_SIZE", 1)])
    out = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(out))
    bench.record_counters(str(tmp_path))
    import json
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    gu = rec["kernels"]["prefill-1t/gate_up"]
    assert gu["launches"] == 2
    assert gu["mfma_flops"] == 2000 * 32768 + 100 * 16384
    assert gu["traffic_bytes"] == (10 + 6) * 1024 * 2.0 + (4 + 1) * 1024 * 1.0
    assert rec["kernels"]["prefill-1t/down"]["mfma_flops"] == 50 * 32768
    assert rec["source_sha256"] == bench.gemm_source_sha()
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(out))
    assert bench.measured_counters("prefill-1t", "gate_up")["launches"] == 2


import pytest  # noqa: E402


@pytest.mark.parametrize("paired,w4a4", [(False, False), (True, False), (False, True)])
def test_cpu_baseline_tiny(paired, w4a4):
    wl = synth.WORKLOADS["tiny"]
    work, dt, threads, sample, phases = bench.cpu_baseline(wl, 1.0, paired, w4a4)
    assert (phases["quantize"] > 0) == w4a4
    assert dt > 0 and threads >= 1 and work > 0
    assert set(phases) >= {"route", "permute", "decode", "gemm", "combine"}
    assert "routed rows" in sample
