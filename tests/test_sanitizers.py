"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/oracle.c) driven through every function with the
  edge cases the parity tests use (tests/native/oracle_check.c).
* The C entry points (csrc/api.hip) and the host launch planning
  (csrc/plan.hip), built as plain C++ with the kernel launchers replaced by
  checking stubs, driven through fixed cases and a seeded sweep of two
  million valid, invalid and extreme argument sets
  (tests/native/abi_host_check.cpp).
A canary with a planted out-of-bounds read and a signed overflow checks that
the sanitizers are really active.  Only gcc/g++ are used: no GPU code is
built here.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sliding_window_learnable_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not available")


def build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def run(exe):
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)


def test_sanitizers_are_active(tmp_path):
    src = tmp_path / "canary.c"
    src.write_text("#include <limits.h>\n#include <stdlib.h>\nint main(int c, char **v) {\n"
                   "  int *a = calloc(2, sizeof(int)); volatile int i = 2; (void)v;\n"
                   "  if (c > 1) { volatile int x = INT_MAX; return x + c; }\n"
                   "  return a[i];\n}\n")
    # each sanitizer on its own, so that the other cannot report the fault first
    asan, ubsan = str(tmp_path / "canary_asan"), str(tmp_path / "canary_ubsan")
    base = [f for f in SAN if not f.startswith("-fsanitize=")]
    build(["gcc", *base, "-fsanitize=address", str(src), "-o", asan])
    build(["gcc", *base, "-fsanitize=undefined", str(src), "-o", ubsan])
    res = run(asan)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr
    res = subprocess.run([ubsan, "x"], capture_output=True, text=True, env=ENV)
    assert res.returncode != 0 and "runtime error" in res.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    build(["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(NATIVE, "oracle_check.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    res = run(exe)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr


def test_entry_points_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    inc = ["-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", *inc,
           "-x", "c++", os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "plan.hip"),
           "-x", "none", os.path.join(NATIVE, "launch_stubs.cpp"),
           os.path.join(NATIVE, "abi_host_check.cpp"), "-o", exe])
    res = run(exe)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr
