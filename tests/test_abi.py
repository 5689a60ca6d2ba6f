"""The C-ABI library loads and exports every entry point include/pa.h declares.

Runs without a GPU: loading libpa.so and resolving symbols makes no HIP call.
"""
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["pa_alloc_pool", "pa_write_kv", "pa_decode", "pa_copy_blocks", "pa_bm_create", "pa_bm_step",
                     "pa_bm_fork", "pa_bm_free_seq", "pa_last_error"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    from paged_kv_cache_355_amd import LIB_PATH
    assert os.path.exists(LIB_PATH), "build libpa.so first (python -m paged_kv_cache_355_amd.build)"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z0-9_]+)\b", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_binding_covers_every_symbol_and_loads():
    from paged_kv_cache_355_amd._lib import SIGNATURES, lib
    assert sorted(SIGNATURES) == declared_functions()
    handle = lib()
    for name in SIGNATURES:
        assert getattr(handle, name) is not None


def test_header_compiles_as_c():
    out = os.path.join("/tmp", "pa_h_check.o")
    src = "#include \"pa.h\"\nint main(void) { return PA_OK; }\n"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-x", "c", "-c", "-",
                    "-o", out], input=src, text=True, check=True)


def test_errors_are_reported_without_a_gpu():
    import paged_kv_cache_355_amd as pk
    with pytest.raises(pk.PaError) as e:
        pk.BlockManager(4, 4, [0, 1, 1, 2])
    assert "permutation" in str(e.value)
    bm = pk.BlockManager(2, 4)
    bm.add_seq(0, 8)
    with pytest.raises(pk.NoBlocksError):
        bm.step([0])
    with pytest.raises(pk.PaError) as e:
        bm.free_seq(7)
    assert e.value.code == -5


def test_pool_takes_both_tensors_or_neither():
    """Caller memory means both K and V; the binding says so before any device work."""
    import torch
    import paged_kv_cache_355_amd as pk
    k = torch.empty((4, 1, 16, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="both k and v"):
        pk.Pool(4, 16, 1, 64, "f16", k=k)
    with pytest.raises(ValueError, match="both k and v"):
        pk.Pool(4, 16, 1, 64, "f16", v=k)
    with pytest.raises(ValueError, match="device tensor"):          # host tensors are refused too
        pk.Pool(4, 16, 1, 64, "f16", k=k, v=k.clone())
