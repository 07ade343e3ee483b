"""Build libgqe.so in-tree for gfx950 with hipcc (no GPU needed to compile).

    python -m sparse_moe_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgqe.so")
BUILD_DIR = os.path.join(HERE, "_build")
# Translation units and their own flags. The projection GEMMs are scheduled
# for instruction-level parallelism (their K loops then overlap the next
# fragment reads with the current MFMAs: Wo 80 -> 65 us at T = 32K); the
# attention kernels keep the default occupancy-first schedule (3% slower
# under the other).
UNITS = [
    ("gqe_api.hip", []),
    ("gemm_launch.hip", ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
]
SRC = os.path.join(CSRC, "gqe_api.hip")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqe.so)")


def _run(cmd, verbose: bool, what: str) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"   # host pass of the fp32 flag
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def _compile_and_link(out: str, flags: list, tag: str, verbose: bool) -> None:
    """Compile every unit with `flags` (+ its own) in parallel, link `out`."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, f"{os.path.splitext(u)[0]}{tag}.o") for u, _ in UNITS]
    jobs = [([hipcc_path(), *flags, *extra, "-c", "-o", o, os.path.join(CSRC, u)], u)
            for (u, extra), o in zip(UNITS, objs)]
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_run, c, verbose, f"hipcc {u}") for c, u in jobs]:
            f.result()
    # the host sanitizers' runtimes are linked too (each -fsanitize= stays behind its -Xarch_host)
    san = [x for i in range(len(flags) - 1) if flags[i] == "-Xarch_host" and flags[i + 1].startswith("-fsanitize=")
           for x in flags[i:i + 2]]
    _run([hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", out, *objs], verbose, "link")


def build(verbose: bool = False) -> str:
    """Compile csrc/ into libgqe.so next to this file; returns its path."""
    tmp = OUT + f".tmp{os.getpid()}"
    _compile_and_link(tmp, HIPCC_FLAGS, "", verbose)
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.remove(tmp)
        raise RuntimeError("hipcc dropped the host side of these kernels (a device-only construct in the "
                           "body failed to compile for the host pass):\n  " + "\n  ".join(missing))
    os.replace(tmp, OUT)
    return OUT


# Host-side sanitizers: AddressSanitizer and UndefinedBehaviorSanitizer on the
# host pass only (each -fsanitize= behind -Xarch_host); the device code is
# built as usual and never runs on the CPU. Used by the CPU tests, which run
# every argument-checking path of the C ABI against this build.
SAN_OUT = os.path.join(HERE, "_build", "libgqe_hostsan.so")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
    # every uninitialised local holds a 0xAA.. pattern instead of whatever the
    # stack held, so a read of one changes the checks' results every time
    "-Xarch_host", "-ftrivial-auto-var-init=pattern",
]


def build_host_sanitized(verbose: bool = False) -> str:
    """libgqe with ASan + UBSan in its host code, at SAN_OUT; returns the path."""
    os.makedirs(os.path.dirname(SAN_OUT), exist_ok=True)
    tmp = SAN_OUT + f".tmp{os.getpid()}"
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS
    _compile_and_link(tmp, flags, "_hostsan", verbose)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


def asan_runtime() -> str:
    """The clang ASan runtime that a non-instrumented host (python) must preload."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc_path())), "..", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if c and os.path.exists(c):
            res = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found")


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
