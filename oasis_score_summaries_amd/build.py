"""Builds liboasis.so (HIP for gfx950) in-tree with hipcc.

Every call compiles every source again: the objects go to ``_build/`` at the
repository root and the shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liboasis.so")
SOURCES = ["abi.cpp", "summaries.hip", "score.hip", "select.hip", "attention.hip", "fused.hip",
           "working_set.hip", "noalloc.hip"]
ARCH = os.environ.get("OASIS_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions are kept out of the device code: ordinary float code
# compiles to scalar VALU and MFMA instructions only.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build liboasis")
    return path


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=(), src_dir: str = CSRC) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(src_dir, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # hipcc's host pass does not know the device-only target feature; that note is noise.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), file=sys.stderr)
    return obj


def build(verbose: bool = False, lib: str = LIB, defines=(), build_dir: str = BUILD,
          src_dir: str = CSRC) -> str:
    """Compile all sources and link the library (default: liboasis.so next to this
    file); ``defines`` are extra -D settings of the kernels' compile-time tunables."""
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{x}" for x in defines]
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra, src_dir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link of liboasis.so failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
