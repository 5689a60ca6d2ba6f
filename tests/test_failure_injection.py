"""Failure paths of the host block manager and the C ABI, forced from the
host (no GPU): each error comes back with its documented code and leaves the
block manager exactly as it was."""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_355_amd as pk
from paged_kv_cache_355_amd._lib import lib

PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_NO_BLOCKS = -1, -2, -3
PA_ERR_NOT_FOUND, PA_ERR_EXISTS = -5, -6


def snapshot(bm, ids):
    return (bm.free_list(), [bm.refcount(b) for b in range(bm.num_blocks)],
            {s: bm.block_table(s) for s in ids}, bm.stats())


def code_of(fn, *args):
    with pytest.raises(pk.PaError) as e:
        fn(*args)
    return e.value.code


def test_each_failure_has_its_code_and_changes_nothing():
    bm = pk.BlockManager(6, 4, [3, 1, 4, 0, 5, 2])
    bm.add_seq(10, 9)            # 3 blocks
    bm.fork(10, 11)              # shares them
    before = snapshot(bm, [10, 11])
    assert code_of(bm.add_seq, 10, 1) == PA_ERR_EXISTS               # duplicate id
    assert code_of(bm.fork, 99, 12) == PA_ERR_NOT_FOUND             # unknown parent
    assert code_of(bm.fork, 10, 11) == PA_ERR_EXISTS                # child id taken
    assert code_of(bm.free_seq, 12) == PA_ERR_NOT_FOUND             # unknown id
    assert code_of(bm.step, [10, 10], 4) == PA_ERR_INVALID          # duplicate ids in one step
    assert code_of(bm.step, [10, 77], 4) == PA_ERR_NOT_FOUND        # unknown id in a step
    assert code_of(bm.add_seq, 12, 13) == PA_ERR_NO_BLOCKS          # needs 4 blocks, 3 free
    assert code_of(bm.append_slot, 12) == PA_ERR_NOT_FOUND
    assert snapshot(bm, [10, 11]) == before
    # a step that cannot finish (both copy-on-write copies need a block, one is left
    # after a third sequence takes two) fails as a whole
    bm.add_seq(12, 8)
    before = snapshot(bm, [10, 11, 12])
    with pytest.raises(pk.NoBlocksError):
        bm.step([10, 11, 12])
    assert snapshot(bm, [10, 11, 12]) == before
    bm.free_seq(11)
    assert code_of(bm.free_seq, 11) == PA_ERR_NOT_FOUND             # double free


def test_c_abi_rejects_bad_arguments():
    L = lib()
    handle = ctypes.c_void_p()
    assert L.pa_bm_create(0, 4, None, ctypes.addressof(handle)) == PA_ERR_INVALID      # no blocks
    assert L.pa_bm_create(8, 4, None, None) == PA_ERR_INVALID                          # no out pointer
    assert L.pa_bm_create(1 << 29, 16, None, ctypes.addressof(handle)) == PA_ERR_INVALID   # slots >= 2^31
    assert L.pa_alloc_pool(16, 4, 1, 96, 1, None, None, ctypes.addressof(handle)) == PA_ERR_UNSUPPORTED  # head_dim
    assert L.pa_alloc_pool(16, 12, 1, 64, 1, None, None, ctypes.addressof(handle)) == PA_ERR_UNSUPPORTED  # block size
    assert L.pa_alloc_pool(16, 4, 1, 64, 7, None, None, ctypes.addressof(handle)) == PA_ERR_UNSUPPORTED   # dtype
    assert L.pa_alloc_pool(1 << 29, 16, 1, 64, 1, None, None, ctypes.addressof(handle)) == PA_ERR_INVALID  # slots >= 2^31
    assert L.pa_write_kv(None, None, None, None, 1, None) == PA_ERR_INVALID          # null pool
    assert L.pa_decode(None, None, 1, None, 1, 1, None, 1, None, 1, ctypes.c_float(0.0), 0, None, 0,
                       None) == PA_ERR_INVALID
    assert L.pa_bm_add_seq(None, 1, 1) == PA_ERR_INVALID
    assert len(L.pa_last_error()) > 0
