"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU builds with gcc/g++; no GPU code is built or run here).

Each driver walks its code over random and corrupted inputs: round trips, bit flips,
truncated containers, buffers too small, malformed tables.  A sanitizer report aborts the
driver, and the test fails with its output.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=gnu11", *SAN, "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "shannonic_oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_tables_and_host_entry_points_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "entropy_coding_quantized_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{os.path.join(ROOT, 'include')}", "-o", exe,
          os.path.join(HERE, "host_driver.cpp"), os.path.join(csrc, "host_tables.cpp"),
          os.path.join(csrc, "api.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV, timeout=600)
    assert "0 failures" in r.stdout
