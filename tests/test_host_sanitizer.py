"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_checks.cpp calls every entry point of include/nk.h on
its validation paths (null pointers, bad sizes and types, windows, split
sizes, workspace shortfalls, the no-allocation call's limit, the planning
queries over extreme sizes, the timing diagnostics).  It is linked with
csrc/api.hip built with the sanitizers on the host side only (the device
code is compiled as usual and never runs) and with stand-ins for the kernel
launchers that abort if reached.  Runs without a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_abi_validation_under_host_sanitizers(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_checks")
    cmd = [cc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "ragged_paged_kv_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi checks: 0 failed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
