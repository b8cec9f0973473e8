"""Build libq4k.so in-tree with hipcc for gfx950.

Usage: python -m quantized_decode_q4_amd.build   (or call build())
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libq4k.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    # keep packed-FP32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, debug_sync: bool | None = None) -> str:
    """Compile libq4k.so. debug_sync (default: environment Q4K_DEBUG_SYNC=1)
    builds the debugging variant in which every call waits for its stream and
    reports a kernel that failed while running as Q4K_ERR_HIP."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if debug_sync is None:
        debug_sync = os.environ.get("Q4K_DEBUG_SYNC", "") == "1"
    tmp = LIB_PATH + ".tmp"
    defs = ["-DQ4K_DEBUG_SYNC"] if debug_sync else []
    cmd = [hipcc, *HIPCC_FLAGS, *defs, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
