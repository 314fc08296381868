"""The host layer (pisa_host.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: compiled with g++ (host code only, no
HIP kernel sources) into tests/abi_host_sanitize.cpp, whose stub launchers
count calls.  Rejected calls must launch nothing and leave sentinel-filled
outputs untouched; valid calls reach one launcher; random problem statements
must not trip either sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "abi_host_sanitize")
    csrc = os.path.join(ROOT, "piecewise_attention_dit_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "pisa_host.cpp"),
           os.path.join(ROOT, "tests", "abi_host_sanitize.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert r.stdout.strip().startswith("OK"), r.stdout
