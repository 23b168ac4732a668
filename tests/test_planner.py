"""The GEMM planner's choices over a sweep of shapes (host logic, no GPU): tests/planner_check.hip is
compiled with hipcc and run on the CPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_planner_choices_are_valid(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "planner_check")
    subprocess.run([hipcc, "-O1", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-o", exe, os.path.join(HERE, "planner_check.hip")], check=True,
                   capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
