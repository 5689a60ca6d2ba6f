"""ctypes declarations for libpa.so (the C ABI in include/pa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same C ABI (for instance a host
# build under the sanitizers); by default the in-tree library.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_NO_BLOCKS = -3
PA_ERR_READ_ONLY = -4
PA_ERR_NOT_FOUND = -5
PA_ERR_EXISTS = -6
PA_ERR_HIP = -7
PA_ERR_NO_MEMORY = -8

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_PARTITION_BALANCED = -1
PA_PARTITION_UNIFORM = -2

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_p = ctypes.c_void_p


class BmStats(ctypes.Structure):
    _fields_ = [
        ("num_blocks", c_i32), ("block_size", c_i32), ("free_blocks", c_i32), ("used_blocks", c_i32),
        ("shared_blocks", c_i32), ("num_seqs", c_i32), ("logical_tokens", c_i64), ("logical_blocks", c_i64),
        ("filled_slots", c_i64), ("cow_copies", c_i64), ("swapped_seqs", c_i32), ("reserved", c_i32),
        ("swapped_tokens", c_i64),
    ]


# name → (restype, argtypes), following include/pa.h.  Every pointer is passed
# as an integer address (c_void_p): torch ``data_ptr()``, numpy
# ``ctypes.data`` or ``ctypes.addressof`` of an output scalar.
SIGNATURES = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_alloc_pool": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p]),
    "pa_free_pool": (None, [c_p]),
    "pa_pool_info": (c_i32, [c_p, c_p, c_p, c_p]),
    "pa_write_kv": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_p]),
    "pa_copy_blocks": (c_i32, [c_p, c_p, c_i32, c_p]),
    "pa_swap_out": (c_i32, [c_p, c_p, c_i32, c_p, c_i64, c_p]),
    "pa_swap_in": (c_i32, [c_p, c_p, c_i32, c_p, c_i64, c_p]),
    "pa_decode_workspace_bytes": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_p]),
    "pa_decode_partition_tokens": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_p]),
    "pa_decode": (c_i32, [c_p, c_p, c_i32, c_p, c_i32, c_i32, c_p, c_i32, c_p, c_i32, ctypes.c_float, c_i32,
                          c_p, c_i64, c_p]),
    "pa_decode_noalloc": (c_i32, [c_p, c_p, c_i32, c_p, c_i32, c_i32, c_p, c_i32, c_p, c_i32, ctypes.c_float, c_i32,
                                  c_p]),
    "pa_decode_append": (c_i32, [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_p, c_i32, c_p, c_i32,
                                 ctypes.c_float, c_i32, c_p, c_i64, c_p]),
    "pa_decode_shared_prefix_workspace_bytes": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_p]),
    "pa_decode_shared_prefix": (c_i32, [c_p, c_p, c_i32, c_p, c_i32, c_i32, c_p, c_i32, c_p, c_i32, ctypes.c_float,
                                        c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_p, c_i64, c_p]),
    "pa_bm_create": (c_i32, [c_i32, c_i32, c_p, c_p]),
    "pa_bm_destroy": (None, [c_p]),
    "pa_bm_add_seq": (c_i32, [c_p, c_i64, c_i32]),
    "pa_bm_fork": (c_i32, [c_p, c_i64, c_i64]),
    "pa_bm_append_slot": (c_i32, [c_p, c_i64, c_p, c_p, c_p]),
    "pa_bm_step": (c_i32, [c_p, c_p, c_i32, c_p, c_p, c_p, c_p, c_i32, c_p]),
    "pa_bm_free_seq": (c_i32, [c_p, c_i64]),
    "pa_bm_block_table": (c_i32, [c_p, c_i64, c_p, c_i32, c_p, c_p]),
    "pa_bm_token_slots": (c_i32, [c_p, c_i64, c_i32, c_i32, c_p]),
    "pa_bm_tables": (c_i32, [c_p, c_p, c_i32, c_p, c_i32, c_p]),
    "pa_bm_dispatch_order": (c_i32, [c_p, c_p, c_i32, c_p]),
    "pa_bm_prefix_groups": (c_i32, [c_p, c_p, c_i32, c_p, c_p, c_p, c_p]),
    "pa_bm_swap_out": (c_i32, [c_p, c_i64, c_p, c_i32, c_p]),
    "pa_bm_swap_in": (c_i32, [c_p, c_i64, c_p, c_i32, c_p]),
    "pa_bm_refcount": (c_i32, [c_p, c_i32, c_p]),
    "pa_bm_free_list": (c_i32, [c_p, c_p, c_i32, c_p]),
    "pa_bm_stats": (c_i32, [c_p, c_p]),
}

_lib = None


class PaError(RuntimeError):
    def __init__(self, code, func, message):
        super().__init__(f"{func} failed ({code}): {message}")
        self.code = code


class NoBlocksError(PaError):
    pass


def lib():
    """The loaded libpa.so with argument types set (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_355_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(code, func):
    if code != PA_OK:
        msg = lib().pa_last_error().decode(errors="replace")
        cls = NoBlocksError if code == PA_ERR_NO_BLOCKS else PaError
        raise cls(code, func, msg)
    return code
