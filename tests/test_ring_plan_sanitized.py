"""The ring drivers' host planning under address and undefined-behaviour sanitizers (CPU only).

Builds the library's pure-host planning code (chunk-table checks, visible-pair
counts, zigzag tables, forward and backward ring plans) together with
tests/sanitize/ring_plan_check.cpp with g++ -fsanitize=address,undefined and
runs it: 1..64 ring steps, 1..8 chunks per table, odd tables, every
steps-per-launch limit, and a happens-before check of every plan's staging
slots (the double buffering of [MLM] section 5), including planted ordering
mistakes that the check must catch; and the kernels' XCD-aware job order
(csrc/cp_job_map.h): one to one onto (block, b*h), each head on one XCD,
key-split pairs on one XCD, head groups of the largest size that fits.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "sanitize", "ring_plan_check.cpp"),
       os.path.join(ROOT, "long_sequence_causal_cp_amd", "csrc", "cp_ring_plan.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_ring_plans_under_sanitizers(tmp_path):
    exe = str(tmp_path / "ring_plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", *SRC, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed" in run.stdout
