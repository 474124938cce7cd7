"""Build libpa.so (gfx950) in-tree with hipcc.

Usage: python -m paged_kv_cache_326_amd.build [-v]

Each HIP source compiles to its own object in parallel, then one link step
produces ``paged_kv_cache_326_amd/libpa.so``.  Packed-fp32 instructions are
disabled for every device pass.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Extra device flags per source.  The 16-bit prefill kernel keeps its matrix
# products' accumulators in ordinary vector registers (LLVM's VGPR form of
# the MFMA instructions): with them in the accumulator file, the compiler
# copies the whole accumulator set around the tile loop's rarely taken
# branches, and every softmax read of the scores becomes a register move.
FILE_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def device_flags(src: str) -> list:
    """hipcc flags for one HIP source of the library."""
    return [*DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libpa.so cannot be built")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):  # host-only C++ (the block manager)
        cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
               "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *device_flags(src), "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


HOST_SANITIZED_LIB = os.path.join(BUILD_DIR, "libpa_host_sanitized.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The library's host C++ alone (block manager, scheduler) as a shared
    library instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts), for running their CPU tests under the sanitizers:
    pa.py loads it when PA_LIB names it, in a process that preloads
    libasan.  No device code is involved."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    cmd = [shutil.which("g++") or "g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           *srcs, "-o", HOST_SANITIZED_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on the host sources:\n{r.stdout}\n{r.stderr}")
    return HOST_SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
