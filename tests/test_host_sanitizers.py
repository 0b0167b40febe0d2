"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): api.hip (argument validation, the split planners, the item order
they model, the status strings) is built for the host with both sanitizers,
with stub kernel launchers, and driven by tests/host_sanitize/driver.cpp
through every validation path and 400 random batches of the planners; the
driver also checks that the kernels' workgroup -> work-unit map covers every
(request, split, row group) once, in range, for a grid of batch shapes.  The
sanitizers instrument host code only; the device side is built as usual and
never runs here."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


def test_api_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "driver")
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", f]
    cmd = [hipcc, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", *host,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(ROOT, "long_context_mla_amd", "csrc", "api.hip"),
           "-x", "hip", os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in out
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
