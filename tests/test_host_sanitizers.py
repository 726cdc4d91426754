"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library is compiled with both sanitizers on its host code (the GPU code object is built but never run)
and linked with tests/host_checks.cpp, which drives every argument check that returns
before a HIP call and a few thousand random and extreme configs. Any sanitizer report or
failed expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_speculative_verification_amd", "csrc")
SOURCES = ["kernels.hip", "tiled.hip", "draft.hip", "api.hip"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], os.path.join(ROOT, "tests", "host_checks.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "host checks: 0 failures" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
