"""Build libgqe.so in-tree for gfx950 with hipcc (no GPU needed to compile).

    python -m sparse_moe_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "gqe_api.hip")
OUT = os.path.join(HERE, "libgqe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqe.so)")


def build(verbose: bool = False) -> str:
    """Compile csrc/ into libgqe.so next to this file; returns its path."""
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [hipcc_path(), *HIPCC_FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"   # host pass of the fp32 flag
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.remove(tmp)
        raise RuntimeError("hipcc dropped the host side of these kernels (a device-only construct in the "
                           "body failed to compile for the host pass):\n  " + "\n  ".join(missing))
    os.replace(tmp, OUT)
    return OUT


def undefined_kernel_stubs(lib: str) -> list[str]:
    """Kernel launch stubs the library references but does not define.

    hipcc's host pass drops a kernel template instance without a diagnostic
    when its body does not compile for the host; the library then links but
    fails to load. An undefined __device_stub__ symbol is that case."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}: {res.stderr}")
    return [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
