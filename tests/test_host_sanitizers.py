"""CPU test: the C ABI's host code (argument validation, split planning,
workspace arithmetic) built with AddressSanitizer and
UndefinedBehaviorSanitizer, its device code unchanged, passes the ABI tests of
tests/test_abi_cpu.py. Any sanitizer report aborts the run."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hostsan():
    path = os.path.join(ROOT, "compact_kv_cache_amd", "_build_hostsan.py")
    spec = importlib.util.spec_from_file_location("_gva_hostsan", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_tests_pass_under_host_sanitizers():
    m = _hostsan()
    try:
        lib = m.build()
        env = m.run_env(lib)
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"sanitized build not possible here: {e}")
    # the sanitized library and the sanitizer runtime are what the child loads
    probe = ("import compact_kv_cache_amd as g; maps = open('/proc/self/maps').read(); "
             "print(g._lib.LIB_PATH); print('asan' in maps and 'libgva_hostsan' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == [lib, "True"], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_cpu.py")], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
