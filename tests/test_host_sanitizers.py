"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

* tests/native/bm_fuzz.cpp drives the C++ block manager (the same source the
  library links) through thousands of random prefill / fork / batched-append /
  release / failing calls, checking refcounts, the free list, table lengths,
  slot placement and copy-on-write pairs after every one.
* The whole host runtime (api.cpp: the C ABI's argument checks, decode
  planning, block-manager wrappers) is built into a library of the same C ABI
  with the device launchers stubbed out (tests/native/device_stubs.cpp), and
  the CPU tests that drive the C ABI run against it (PA_LIBRARY) with the
  sanitizer runtime preloaded into Python.

Both are built here with g++ (host code only; no GPU).
"""
import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_355_amd", "csrc")
HIP_LIB = "/opt/rocm/lib/libamdhip64.so"
ABI_TESTS = ["tests/test_abi.py", "tests/test_block_manager_parity.py", "tests/test_decode_plan.py",
             "tests/test_failure_injection.py"]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "bm_fuzz")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-static-libasan",
                    "-fno-sanitize-recover=undefined", "-I", CSRC, os.path.join(ROOT, "tests", "native", "bm_fuzz.cpp"),
                    os.path.join(CSRC, "block_manager.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe, "4000"], capture_output=True, text=True, env=env, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 failed checks" in out.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(HIP_LIB), reason="needs g++ and the HIP runtime")
def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "libpa_host_asan.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "block_manager.cpp"),
                    os.path.join(ROOT, "tests", "native", "device_stubs.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", so], check=True)
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    env = dict(os.environ, PA_LIBRARY=so, LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # -s: a sanitizer report ends the process at once; uncaptured, it reaches the pipe
    out = subprocess.run([sys.executable, "-m", "pytest", *ABI_TESTS, "-q", "-s", "-p", "no:cacheprovider"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert out.returncode == 0, out.stdout[-4000:] + out.stderr[-4000:]
    assert "runtime error" not in out.stdout + out.stderr
