"""Host-sanitized build of the GVA library, for the CPU test suite.

The C ABI layer (csrc/api.hip: argument validation, split planning, workspace
arithmetic, dispatch) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code only; its device code and the
kernel sources are built exactly as in _build.py. The result,
_build/libgva_hostsan.so, is loaded in place of libgva.so by setting
GVA_LIBRARY, with the sanitizer runtime preloaded (run_env() gives the
environment). Nothing here is used on a GPU: the sanitized library serves
the host-only validation tests.

Run as `python compact_kv_cache_amd/_build_hostsan.py`.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def _build_module():
    spec = importlib.util.spec_from_file_location("_gva_build", os.path.join(PKG, "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# Each sanitizer flag is passed to the host compilation only (-Xarch_host
# right before it), so the gfx950 code objects are the ordinary ones.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """Path of the AddressSanitizer runtime of ROCm's clang (it carries the
    UndefinedBehaviorSanitizer handlers as well)."""
    b = _build_module()
    clang = os.path.join(os.path.dirname(os.path.realpath(b._hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError(f"AddressSanitizer runtime not found (clang printed {out!r})")
    return out


def build(verbose: bool = False) -> str:
    b = _build_module()
    os.makedirs(b.OUT_DIR, exist_ok=True)
    api = os.path.join(b.CSRC, "api.hip")
    obj = os.path.join(b.OUT_DIR, "api.hostsan.o")
    cmd = [b._hipcc(), "-O1", "-g", *[f for f in b.COMMON if f != "-O3"], *b.DEVICE_FLAGS, *HOST_SANITIZE,
           "-c", api, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    # the kernel objects of the ordinary build (compiled here if missing)
    others = []
    for src in sorted(os.listdir(b.CSRC)):
        if not src.endswith(".hip") or src == "api.hip":
            continue
        o = os.path.join(b.OUT_DIR, src + ".o")
        if not os.path.exists(o) or os.path.getmtime(o) < os.path.getmtime(os.path.join(b.CSRC, src)):
            o = b._compile(os.path.join(b.CSRC, src))
        others.append(o)
    lib = os.path.join(b.OUT_DIR, "libgva_hostsan.so")
    cmd = [b._hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_SANITIZE, "-shared-libasan",
           "-o", lib, obj, *others]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


def run_env(lib: str) -> dict:
    """Environment that loads `lib` as the GVA library under the sanitizers:
    any report aborts the process (leak checking is off: the interpreter
    itself is not instrumented)."""
    env = dict(os.environ)
    env["GVA_LIBRARY"] = lib
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    path = build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "test":
        root = os.path.dirname(PKG)
        sys.exit(subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                                 os.path.join(root, "tests", "test_abi_cpu.py")], env=run_env(path),
                                cwd=root).returncode)
