"""Build the HIP C-ABI library libssa.so in-tree for gfx950.

`build()` always recompiles (hipcc cross-compiles without a GPU). The
library is written next to this file, where the ctypes binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libssa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["ssa_kernel.hip", "ssa_host.cpp", "ssa_gate.cpp", "ssa_calib.cpp"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for every HIP translation unit.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile the HIP kernels and the host sources into libssa.so; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


HOST_SOURCES = ["ssa_host.cpp", "ssa_gate.cpp", "ssa_calib.cpp"]


def build_host_check(out_path: str, verbose: bool = False) -> str:
    """CPU-only build of the host library for the sanitizer tests: the host
    sources under AddressSanitizer and UndefinedBehaviorSanitizer (g++), with
    the kernel launchers replaced by ssa_launch_check.cpp, which checks the
    planned launches against the caller's buffer extents instead of launching.
    Load it into a process started with the ASan runtime preloaded."""
    cxx = shutil.which("g++") or "/usr/bin/g++"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES + ["ssa_launch_check.cpp"]], "-o", out_path]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
