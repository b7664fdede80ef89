"""The C-ABI refusal layer under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host/abi_sanitize.cpp includes qsa_abi.hip's host code with stub kernel
launchers (they check the invariants the kernels rely on and touch no device
memory) and sweeps every entry point over valid, refused and extreme argument
combinations.  Built with g++ and the host sanitizers; no GPU involved.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "abi_sanitize.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_layer_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "abi_sanitize"
    inc = "/opt/rocm/include"
    build = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", inc, SRC, "-o", str(exe)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr, r.stderr[-4000:]
