"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): tests/host_checks/abi_checks.cpp is built with the library's sources, the sanitizers
on the host code only, and run; it feeds every size query edge values of every shape field
and calls each entry point with arguments its checks must reject (no kernel is launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "branch_folding_amd", "csrc")
from branch_folding_amd.build import SOURCES  # noqa: E402  (the library's own source list)
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


@pytest.mark.timeout(600)
def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", "-w",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include")]
    for f in SANITIZE:            # host code only: the device code is built as usual
        cmd += ["-Xarch_host", f]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += [os.path.join(ROOT, "tests", "host_checks", "abi_checks.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "OK: 0 failure(s)" in out, out[-4000:]
