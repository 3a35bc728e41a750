"""CPU debug build of the library's host code (bounds assertions + address and
undefined-behaviour sanitizers): validation, workspace layout, the store's chunk map, the
bucket scan and block table, and the expert cache policy, run on the host
(tests/csrc/host_checks.cpp).  No GPU needed."""
import os
import shutil
import subprocess

import pytest

from quantized_moe_router_amd import build as B


@pytest.mark.skipif(not (os.environ.get("HIPCC") or os.path.exists("/opt/rocm/bin/hipcc")
                         or shutil.which("hipcc")), reason="hipcc not installed")
def test_host_debug_build_passes_its_bounds_checks():
    exe = B.build_host_checks()
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks: ok" in r.stdout
