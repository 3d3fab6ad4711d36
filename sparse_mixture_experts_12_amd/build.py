"""Build libmoe.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc, and
libmoe_probe.so (the roofline probes bench.py --probe times; not part of the
layer).

Every source compiles to its own object in parallel (each carries its own
gfx950 code object), then hipcc links the shared library."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
PROBE_SRC = os.path.join(PKG, "csrc", "probe", "roofline_probe.hip")
OBJ_DIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd[-3:])}")


def build(verbose: bool = False, out: str = LIB, extra=(), jobs: int = 0) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(OBJ_DIR, f"{tag}.{os.path.splitext(os.path.basename(src))[0]}.o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
    workers = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False, out: str = PROBE_LIB) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
