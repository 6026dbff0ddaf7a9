"""Compile the HIP sources of the GVA library into libgva.so (gfx950), and the
benchmark's measurement kernels (bench_kernels/) into libgva_ceiling.so.

Run as `python compact_kv_cache_amd/_build.py` or through
`__graft_entry__.build()` (both load this file without importing the package,
whose import needs the library). Every call recompiles; objects go to
compact_kv_cache_amd/_build/, the library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgva.so")
ARCH = os.environ.get("GVA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the device code: hipcc would emit
# them from ordinary float code otherwise.
# The atomic optimizer is off: every atomic here is issued by one lane, and its
# wave-aggregated rewrite reads the result back at once, which makes the wave
# wait for all of its earlier loads (the tile stream) right after the atomic.
# Kernel-argument preloading: the leading scalar arguments of a kernel (up to
# 14 dwords beside the argument pointer) arrive in scalar registers at wave
# launch instead of through a memory fetch; code objects keep a fallback entry
# that loads them for firmware without the feature.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                "-mllvm", "-amdgpu-kernarg-preload-count=16"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the GVA library needs ROCm's hipcc to build")


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


BENCH_SRC = os.path.join(PKG, "bench_kernels")
CEILING_LIB = os.path.join(PKG, "libgva_ceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """The benchmark's measurement kernels (empty launch, plain reads):
    libgva_ceiling.so, separate from the GVA library."""
    srcs = sorted(glob.glob(os.path.join(BENCH_SRC, "*.hip")))
    objs = [_compile(src) for src in srcs]
    tmp = CEILING_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print(f"built {CEILING_LIB}")
    return CEILING_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_ceiling(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
