"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only). Builds libgqe with both sanitizers on its host pass, then runs
every test of tests/test_abi.py (each argument check and status code of every
entry point, before any HIP call) against that build in a child process with
the ASan runtime preloaded. Any sanitizer report ends the child with an error
and fails this test."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from sparse_moe_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    lib = B.build_host_sanitized()
    log = str(tmp_path / "san")
    env = dict(os.environ)
    env.update(GQE_LIB_PATH=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    reports = "".join(open(p).read() for p in sorted(glob.glob(log + "*")))
    assert res.returncode == 0 and not reports, (res.stdout[-3000:], res.stderr[-3000:], reports[:6000])
    assert " passed" in res.stdout
