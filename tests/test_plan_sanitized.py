"""The planner under AddressSanitizer and UndefinedBehaviorSanitizer: tests/plan_fuzz.cpp
and csrc/plan.cpp built with g++ (host code only, no GPU) and run over random shapes,
including the largest the interface takes, and random forced options."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "row_normalization_norm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", CSRC, os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe, "2000000"], capture_output=True, text=True, timeout=600,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    ok, refused = (int(v) for v in r.stdout.split()[1::2])
    assert ok > 500000 and refused > 0, r.stdout
