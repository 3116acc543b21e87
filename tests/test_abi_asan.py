"""The C ABI's host code under AddressSanitizer, without a GPU: the library's sources are
built with host-side ASan (device code as usual) into a small driver, tests/asan_driver.cpp,
that runs every path before a launch -- validation of every entry point, workspace sizes,
segment plans, status strings, profiling buckets -- over a grid of valid and invalid
shapes. Any ASan report or failed check fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

from gated_delta_rule_depthwise_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the driver")
def test_host_code_under_asan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "asan_driver")
        cmd = [lib_build.hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # sanitizers on the host code only
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
               "-I", lib_build.CSRC] + lib_build.SOURCES + [
               os.path.join(ROOT, "tests", "asan_driver.cpp"), "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        out = run.stdout + run.stderr
        assert "AddressSanitizer" not in out, out[-4000:]
        assert run.returncode == 0, out[-4000:]
        assert "0 of" in run.stdout, out[-2000:]
