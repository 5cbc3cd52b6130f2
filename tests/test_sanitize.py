"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The oracle's C (oracle/kda_oracle.c), linked with tests/sanitize/oracle_checks.c
  by gcc with the sanitizers: forwards over ragged and empty packed sequences, head
  and column selections, decode against forward, the backward, the DPLR forward and
  the rejections.
- The library's host layer (the C ABI's checks, workspace sizing, status strings,
  timing bookkeeping), built by hipcc with the sanitizers on the host pass only and
  driven by tests/sanitize/abi_host_checks.c through every path that returns before
  a HIP call, so no GPU is needed.
Leak detection is on. The builds go to _build/sanitize/ and are redone when a
source is newer."""
import os
import shutil
import subprocess

import pytest

from gated_delta_rule_57_amd import build as kbuild
from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def stale(target, sources):
    return not os.path.exists(target) or any(os.path.getmtime(s) > os.path.getmtime(target) for s in sources)


def run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 failures" in out, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    driver = os.path.join(HERE, "oracle_checks.c")
    if stale(exe, [driver, obuild.oracle_source_path()]):
        obuild.build_sanitized_program(driver, exe)
    run(exe)


@pytest.mark.timeout(600)
def test_library_host_layer_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libkda_asan.so")
    srcs = [os.path.join(kbuild.CSRC, s) for s in os.listdir(kbuild.CSRC)] + [os.path.join(ROOT, "include", "kda.h")]
    if stale(lib, srcs):
        kbuild.build_host_sanitized(lib)
    exe = os.path.join(OUT, "abi_host_checks")
    driver = os.path.join(HERE, "abi_host_checks.c")
    rt = kbuild.sanitizer_runtime_dir()
    if stale(exe, [driver, lib]):
        clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
        subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", "-shared-libsan", "-o", exe, driver, "-L" + OUT, "-lkda_asan",
                        "-Wl,-rpath," + OUT, "-Wl,-rpath," + rt], check=True)
    run(exe)
