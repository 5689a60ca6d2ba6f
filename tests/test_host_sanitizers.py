"""The host block manager under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/bm_fuzz.cpp drives the C++ block manager (the same source the
library links) through thousands of random prefill / fork / batched-append /
release / failing calls, checking refcounts, the free list, table lengths,
slot placement and copy-on-write pairs after every one.  It is built here
with g++ and the sanitizers (host code only; no GPU).
"""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_355_amd", "csrc")


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
