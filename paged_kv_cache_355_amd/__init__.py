"""MI355X-native paged KV cache and paged decode attention.

The work is done by libpa.so (HIP kernels for gfx950 plus a C++ host block
manager, C ABI in include/pa.h); this package is its thin Python binding.
The library is loaded on first use and its absence is an error: nothing here
falls back to another implementation.
"""
from ._lib import PaError, NoBlocksError, LIB_PATH, lib, PA_PARTITION_BALANCED, PA_PARTITION_UNIFORM
from .api import (Pool, BlockManager, write_kv, copy_blocks, swap_out, swap_in, decode, decode_workspace_bytes,
                  decode_partition_tokens, decode_noalloc, decode_shared_prefix,
                  decode_shared_prefix_workspace_bytes, torch_dtype, dtype_name)

__all__ = ["PaError", "NoBlocksError", "LIB_PATH", "lib", "PA_PARTITION_BALANCED", "PA_PARTITION_UNIFORM", "Pool",
           "BlockManager", "write_kv", "copy_blocks", "swap_out", "swap_in", "decode", "decode_workspace_bytes",
           "decode_partition_tokens", "decode_noalloc", "decode_shared_prefix",
           "decode_shared_prefix_workspace_bytes", "torch_dtype", "dtype_name"]
