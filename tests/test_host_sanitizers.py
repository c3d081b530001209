"""The C ABI's host side under the address and undefined-behaviour
sanitizers, on the CPU.

host.cpp (validation, the execution plan and workspace sizing, the host
index check, every extern "C" entry point) is plain C++ with no HIP.  This
test builds it with g++ -fsanitize=address,undefined, links the launcher
stand-ins of tests/host_stubs.cpp in place of the HIP kernels, and runs the
boundary tests (including the fuzzed-argument test) against that library in
a child process with the ASan runtime preloaded.  Any sanitizer report
aborts the child and fails this test.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qkv_norm_rope_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None,
                                reason="needs g++ with the sanitizer runtimes")


def _asan_runtime() -> str:
    out = subprocess.run(["g++", "-print-file-name=libasan.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else ""


def test_boundary_under_asan_ubsan(tmp_path):
    asan = _asan_runtime()
    if not asan:
        pytest.skip("libasan.so not found")
    lib = tmp_path / "libqkvnr_host_san.so"
    cmd = ["g++", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "host.cpp"),
           os.path.join(ROOT, "tests", "host_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_PRELOAD=asan, QKVNR_LIBRARY=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_boundary.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
