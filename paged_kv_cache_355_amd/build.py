"""Build libpa.so (HIP kernels for gfx950 + the C-ABI host runtime) in-tree.

Run as ``python -m paged_kv_cache_355_amd.build`` or through
``__graft_entry__.build()``.  Every call recompiles.  Objects go to
``_build/`` at the repository root; the library lands next to this file.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed-FP32 VALU forms are disabled.
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]

SOURCES = [
    ("kv_kernels.hip", True),
    ("scratch.hip", True),
    ("decode_f32.hip", True),
    ("decode_f16.hip", True),
    ("decode_bf16.hip", True),
    ("api.cpp", False),
    ("block_manager.cpp", False),
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{proc.stdout}")
    return proc.stdout


def _compile(src, device):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *(DEVICE if device else ["-D__HIP_PLATFORM_AMD__"]), "-c", os.path.join(CSRC, src),
           "-o", obj]
    out = _run(cmd)
    return obj, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda sd: _compile(*sd), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for o, out in results:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
