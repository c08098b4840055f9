"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/abi_sanitize/driver.cpp links csrc/api.hip (compiled with host-only sanitizers; the device
side of the file is only the allocation-free entry point's scratch array) against stub kernel
launchers, and calls every entry point with valid arguments (a launch is requested), invalid ones
(the documented status, nothing launched) and extreme sizes (the overflow guards). No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           # sanitizers on the host code only
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "ternary_weight_quantized_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "abi_sanitize", "driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env, cwd=str(tmp_path))
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "0 failures" in out and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
