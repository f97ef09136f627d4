"""Build the HIP library (gfx950) in-tree: top_routing_dispatch_amd/libmoe_hip.so.

Every .hip source under csrc/ is compiled to an object with hipcc, in
parallel, then linked into one shared library.  Cross-compiles without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # packed-FP32 instructions are kept out of the device code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass reports the device-only target feature as unknown: harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8, out: str = LIB_PATH, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link `out` (the in-tree library by default;
    `defines` and another `out` / `build_dir` give a variant build for
    kernel-tuning experiments, loaded through MOE_LIB_PATH)."""
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        log = _run([HIPCC, *FLAGS, *dflags, "-c", src, "-o", obj])
        if verbose and log.strip():
            print(log)
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
