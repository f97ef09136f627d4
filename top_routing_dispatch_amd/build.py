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


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
# sanitizer flags go to the host pass only (device code is built as usual),
# and the objects are linked by the host compiler against the shared
# sanitizer runtime, which the process must preload
# (LD_PRELOAD=sanitizer_runtime()).
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_hip_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANGXX = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm compiler (it carries
    the UndefinedBehaviorSanitizer handlers too)."""
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not found:
        raise RuntimeError("no AddressSanitizer runtime under /opt/rocm/llvm")
    return sorted(found)[-1]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                      [os.path.join(INCLUDE, "moe.h")]):
        with open(src, "rb") as f:
            h.update(os.path.basename(src).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def build_sanitized(verbose: bool = False, jobs: int = 8) -> str:
    """The library with its host code under ASan + UBSan (-O1 -g), in
    _build/san; rebuilt only when a source changed since the last build."""
    os.makedirs(SAN_DIR, exist_ok=True)
    stamp = os.path.join(SAN_DIR, "sources_digest")
    digest = sources_digest()
    if os.path.exists(SAN_LIB) and os.path.exists(stamp) and open(stamp).read().strip() == digest:
        return SAN_LIB
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = [f if f != "-O3" else "-O1" for f in FLAGS] + ["-g"] + SAN_FLAGS

    def compile_one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = SAN_LIB + ".tmp"
    _run([CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libsan", *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp])
    os.replace(tmp, SAN_LIB)
    with open(stamp, "w") as f:
        f.write(digest + "\n")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
