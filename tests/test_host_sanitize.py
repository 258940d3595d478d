"""The C ABI's host code (argument checks, the part rule, the planner and its
row chunks, workspace sizes, the tuner's table, the no-allocation schedule)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
driven over many shapes, forced plans and bad arguments
(tests/host_sanitize/driver.cpp), with the kernel launchers and the HIP
runtime calls replaced by host stand-ins (stubs.cpp).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
GXX = shutil.which("g++")
HIP_INC = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(GXX is None or not os.path.isdir(HIP_INC), reason="g++ or the HIP headers missing")


def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    srcs = [os.path.join(ROOT, "linear_exl3_input_amd", "csrc", "exl3_host.cpp"),
            os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")]
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC, "-I", os.path.join(ROOT, "include"),
           *srcs, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert "host checks done: 0 failures" in r.stdout
