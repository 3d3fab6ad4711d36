"""Build libmoe.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmoe.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
