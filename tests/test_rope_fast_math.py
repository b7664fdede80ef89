"""The kernels' f32 rotary cos/sin and the certificate that lets its bf16
rounding stand in for the double evaluation (qsa_rope_math.h), checked on
the CPU: over every position below 262147 at four rotary tables, and over
every non-negative f32 angle below 2^18: error below half the allowance,
and no certified value differing from the bf16 rounding of the f32 rounding
of double cos/sin.  Same IEEE operations as on the GPU (FMA,
round-to-even, no contraction)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_f32_rope_trig_certificate_holds_on_every_position(tmp_path):
    exe = tmp_path / "rope_f32_check"
    src = os.path.join(ROOT, "tests", "host", "rope_f32_check.cpp")
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " wrong 0" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_f32_rope_trig_certificate_holds_on_every_f32_angle(tmp_path):
    """Every non-negative f32 angle below 2^18 (about 1.2e9 of them, any
    rotary table and position the kernels can meet): the certificate never
    accepts a value whose bf16 differs from the double reading's, and the
    single-precision error stays below half its allowance."""
    exe = tmp_path / "rope_f32_exhaustive"
    src = os.path.join(ROOT, "tests", "host", "rope_f32_exhaustive.cpp")
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-pthread", src, "-o",
                        str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    threads = str(max(1, min(16, os.cpu_count() or 1)))
    r = subprocess.run([str(exe), threads], capture_output=True, text=True, timeout=1200)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " wrong 0" in r.stdout
