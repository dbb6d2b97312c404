"""The library's host layer (argument checks, status strings, error detail)
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/abi_checks.c through every entry point's rejection paths.  CPU only:
no call reaches the GPU."""
import os
import subprocess

import pytest


def test_host_checks_under_asan_and_ubsan(tmp_path):
    from sparse_fp4_expert_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    exe = build.build_host_checker(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "ok: 0 failure(s)" in r.stdout, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
