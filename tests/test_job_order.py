"""The attention-backward workgroup order (bwd_job in csrc/backward.hpp),
checked on the CPU: a host program built from the same header with hipcc
issues the order for about 2,000 shapes (ragged lengths, 1-10 groups, up to 8
sequences, with and without the shared head's group) and checks that every
job is issued exactly once and that work decreases along the order."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_attention_amd", "csrc")


@pytest.mark.timeout(300)
def test_backward_job_order_is_a_decreasing_bijection(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "job_order_check")
    src = os.path.join(ROOT, "tests", "cpp", "job_order_check.cpp")
    b = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, "-I",
                        os.path.join(ROOT, "include"), "-o", exe, src], capture_output=True, text=True, timeout=240)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-3000:]
