"""Host-side sanitizer runs (CPU only, no GPU needed).

- The oracle (oracle/q4_oracle.c) built by gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer, driven through every function on small
  inputs and edge cases by tests/sanitize/oracle_driver.c.
- The library's host code (argument checks, queue, capture, mailbox,
  workspace bookkeeping) built with the same sanitizers (device code
  unchanged), with the ABI test module run against it in a subprocess that
  preloads clang's sanitizer runtime.  The export-list test is left out of
  that run: a sanitized build exports a few extra C++ helpers.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "_build", "sanitize")
# host-only sanitizer flags for hipcc (each one behind -Xarch_host)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def test_oracle_under_address_and_undefined_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
                    os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "q4_oracle.c"),
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle driver: ok" in res.stdout


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_library_host_checks_under_address_and_undefined_sanitizers():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or clang's sanitizer runtime not found")
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_q4mv_build", os.path.join(ROOT, "affine_q4_matvec_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    os.makedirs(BUILD, exist_ok=True)
    lib = b.build(out=os.path.join(BUILD, "libq4mv.so"), extra_flags=HOST_SANITIZE)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", Q4MV_TEST_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          "-k", "not test_only_the_c_abi_is_exported"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
