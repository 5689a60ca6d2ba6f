"""Thin Python binding over libpa.so: argument marshalling only.

Every computation runs in the library (HIP kernels for the device calls,
C++ for the block manager).  PyTorch supplies device memory and the HIP
stream; numpy arrays carry block-manager outputs on the host.
"""
import ctypes

import numpy as np

from ._lib import lib, check, BmStats, PA_F32, PA_F16, PA_BF16

DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def dtype_name(torch_dt):
    import torch
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[torch_dt]


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev_ptr(t, what, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


# ----------------------------------------------------------------------------
# pool
# ----------------------------------------------------------------------------
class Pool:
    """A paged KV pool; K and V are torch tensors [num_blocks][kv_heads][block_size][head_dim]."""

    def __init__(self, num_blocks, block_size, kv_heads, head_dim, dtype, device=None, k=None, v=None):
        import torch
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.kv_heads, self.head_dim, self.dtype = int(kv_heads), int(head_dim), dtype
        shape = (self.num_blocks, self.kv_heads, self.block_size, self.head_dim)
        tdt = torch_dtype(dtype)
        if (k is None) != (v is None):
            raise ValueError("pass both k and v (caller memory) or neither (allocated here)")
        if k is None:
            device = device or "cuda"
            k = torch.empty(shape, dtype=tdt, device=device)
            v = torch.empty(shape, dtype=tdt, device=device)
        self.k, self.v = k, v
        handle = ctypes.c_void_p()
        check(lib().pa_alloc_pool(self.num_blocks, self.block_size, self.kv_heads, self.head_dim,
                                  DTYPE_CODES[dtype], _dev_ptr(k, "k", tdt, shape), _dev_ptr(v, "v", tdt, shape),
                                  ctypes.addressof(handle)), "pa_alloc_pool")
        self.handle = handle.value

    @property
    def block_bytes(self):
        return self.kv_heads * self.block_size * self.head_dim * ELEM_BYTES[self.dtype]

    def close(self):
        if getattr(self, "handle", None):
            lib().pa_free_pool(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def write_kv(pool, k_new, v_new, slot_mapping, stream=None):
    """Scatter rows k_new/v_new [n][kv_heads][head_dim] into their slots (−1 = skip)."""
    import torch
    n = int(slot_mapping.shape[0])
    shape = (n, pool.kv_heads, pool.head_dim)
    tdt = torch_dtype(pool.dtype)
    check(lib().pa_write_kv(pool.handle, _dev_ptr(k_new, "k_new", tdt, shape), _dev_ptr(v_new, "v_new", tdt, shape),
                            _dev_ptr(slot_mapping, "slot_mapping", torch.int32), n, _stream(stream)), "pa_write_kv")


def copy_blocks(pool, pairs, stream=None):
    """Copy whole blocks for each (src, dst) row of the int32 device tensor ``pairs``."""
    import torch
    n = int(pairs.shape[0])
    if n == 0:
        return
    check(lib().pa_copy_blocks(pool.handle, _dev_ptr(pairs, "pairs", torch.int32, (n, 2)), n, _stream(stream)),
          "pa_copy_blocks")


def _swap(pool, blocks, host, out, stream):
    import torch
    n = int(blocks.shape[0])
    if n == 0:
        return
    if host.device.type != "cpu" or not host.is_pinned() or not host.is_contiguous():
        raise ValueError("host must be a contiguous pinned CPU tensor (pin_memory=True)")
    nbytes = host.numel() * host.element_size()
    fn = lib().pa_swap_out if out else lib().pa_swap_in
    check(fn(pool.handle, _dev_ptr(blocks, "blocks", torch.int32, (n,)), n, host.data_ptr(), nbytes, _stream(stream)),
          "pa_swap_out" if out else "pa_swap_in")


def swap_out(pool, blocks, host, stream=None):
    """Copy pool blocks (int32 device tensor) to a pinned host tensor laid out
    [n][2][block_bytes] (K tile, then V tile, of each block)."""
    _swap(pool, blocks, host, True, stream)


def swap_in(pool, blocks, host, stream=None):
    """Copy a pinned host tensor laid out as ``swap_out`` writes it into pool blocks."""
    _swap(pool, blocks, host, False, stream)


def decode_workspace_bytes(pool, num_seqs, q_heads, max_context_len, partition_tokens=0):
    """Workspace bytes ``decode`` needs; a new workspace must be zero-filled once before use."""
    out = ctypes.c_int64()
    check(lib().pa_decode_workspace_bytes(pool.handle, num_seqs, q_heads, max_context_len, partition_tokens,
                                          ctypes.addressof(out)), "pa_decode_workspace_bytes")
    return out.value


def decode_partition_tokens(pool, num_seqs, q_heads, max_context_len, partition_tokens=0):
    """Partition length ``decode`` will use (PA_PARTITION_BALANCED = -1 for the balanced split,
    PA_PARTITION_UNIFORM = -2 for the uniform split)."""
    out = ctypes.c_int32()
    check(lib().pa_decode_partition_tokens(pool.handle, num_seqs, q_heads, max_context_len, partition_tokens,
                                           ctypes.addressof(out)), "pa_decode_partition_tokens")
    return out.value


def decode(pool, q, block_tables, context_lens, max_context_len, out=None, out_dtype=None, scale=None,
           partition_tokens=0, workspace=None, stream=None, append=None):
    """Paged decode attention; returns ``out`` [num_seqs][q_heads][head_dim].
    ``append=(k_new, v_new, slot_mapping)`` runs pa_decode_append: each
    sequence's new token (its last, row s of k_new/v_new) is written into
    its slot in the same launch, as pa_write_kv would, before it is attended."""
    import torch
    num_seqs, q_heads, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    tdt = torch_dtype(pool.dtype)
    odt = out_dtype or pool.dtype
    if out is None:
        out = torch.empty((num_seqs, q_heads, d), dtype=torch_dtype(odt), device=q.device)
    ws_bytes = decode_workspace_bytes(pool, num_seqs, q_heads, max_context_len, partition_tokens)
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)   # merge counters start at zero
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stride = int(block_tables.shape[1]) if block_tables.dim() == 2 else 0
    args = (_dev_ptr(out, "out", torch_dtype(odt), (num_seqs, q_heads, d)), DTYPE_CODES[odt], _dev_ptr(q, "q", tdt),
            num_seqs, q_heads, _dev_ptr(block_tables, "block_tables", torch.int32), stride,
            _dev_ptr(context_lens, "context_lens", torch.int32, (num_seqs,)), int(max_context_len),
            float(scale) if scale else 0.0, int(partition_tokens), ws_ptr, ws_len, _stream(stream))
    if append is None:
        check(lib().pa_decode(pool.handle, *args), "pa_decode")
    else:
        k_new, v_new, slot_mapping = append
        shape = (num_seqs, pool.kv_heads, pool.head_dim)
        check(lib().pa_decode_append(pool.handle, _dev_ptr(k_new, "k_new", tdt, shape),
                                     _dev_ptr(v_new, "v_new", tdt, shape),
                                     _dev_ptr(slot_mapping, "slot_mapping", torch.int32, (num_seqs,)), *args),
              "pa_decode_append")
    return out


def decode_noalloc(pool, q, block_tables, context_lens, max_context_len, out=None, out_dtype=None, scale=None,
                   partition_tokens=0, stream=None):
    """``decode`` without a workspace (pa_decode_noalloc): partial results go
    to the library's static per-GPU array; ``out`` is the only buffer used.
    Calls that may overlap on one GPU must be serialised."""
    import torch
    num_seqs, q_heads, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    odt = out_dtype or pool.dtype
    if out is None:
        out = torch.empty((num_seqs, q_heads, d), dtype=torch_dtype(odt), device=q.device)
    stride = int(block_tables.shape[1]) if block_tables.dim() == 2 else 0
    check(lib().pa_decode_noalloc(
        pool.handle, _dev_ptr(out, "out", torch_dtype(odt), (num_seqs, q_heads, d)), DTYPE_CODES[odt],
        _dev_ptr(q, "q", torch_dtype(pool.dtype)), num_seqs, q_heads,
        _dev_ptr(block_tables, "block_tables", torch.int32), stride,
        _dev_ptr(context_lens, "context_lens", torch.int32, (num_seqs,)), int(max_context_len),
        float(scale) if scale else 0.0, int(partition_tokens), _stream(stream)), "pa_decode_noalloc")
    return out


def decode_shared_prefix_workspace_bytes(pool, num_seqs, q_heads, max_context_len, max_prefix_tokens,
                                         partition_tokens=0):
    """Workspace bytes ``decode_shared_prefix`` needs."""
    out = ctypes.c_int64()
    check(lib().pa_decode_shared_prefix_workspace_bytes(pool.handle, num_seqs, q_heads, max_context_len,
                                                        max_prefix_tokens, partition_tokens, ctypes.addressof(out)),
          "pa_decode_shared_prefix_workspace_bytes")
    return out.value


def decode_shared_prefix(pool, q, block_tables, context_lens, max_context_len, group_start, prefix_tokens,
                         max_group_size, max_prefix_tokens, out=None, out_dtype=None, scale=None, partition_tokens=0,
                         workspace=None, stream=None):
    """Sharing-aware paged decode (each group's common prefix read once per
    kv-head); ``group_start`` [num_groups + 1] and ``prefix_tokens``
    [num_seqs] are int32 device tensors (see ``BlockManager.prefix_groups``)."""
    import torch
    num_seqs, q_heads, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    tdt = torch_dtype(pool.dtype)
    odt = out_dtype or pool.dtype
    if out is None:
        out = torch.empty((num_seqs, q_heads, d), dtype=torch_dtype(odt), device=q.device)
    ws_bytes = decode_shared_prefix_workspace_bytes(pool, num_seqs, q_heads, max_context_len, max_prefix_tokens,
                                                    partition_tokens)
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stride = int(block_tables.shape[1]) if block_tables.dim() == 2 else 0
    num_groups = int(group_start.numel()) - 1
    check(lib().pa_decode_shared_prefix(
        pool.handle, _dev_ptr(out, "out", torch_dtype(odt), (num_seqs, q_heads, d)), DTYPE_CODES[odt],
        _dev_ptr(q, "q", tdt), num_seqs, q_heads, _dev_ptr(block_tables, "block_tables", torch.int32), stride,
        _dev_ptr(context_lens, "context_lens", torch.int32, (num_seqs,)), int(max_context_len),
        float(scale) if scale else 0.0, num_groups,
        _dev_ptr(group_start, "group_start", torch.int32, (num_groups + 1,)) if num_groups > 0 else None,
        _dev_ptr(prefix_tokens, "prefix_tokens", torch.int32, (num_seqs,)) if num_groups > 0 else None,
        int(max_group_size), int(max_prefix_tokens), int(partition_tokens), ws_ptr, ws_len, _stream(stream)),
        "pa_decode_shared_prefix")
    return out


# ----------------------------------------------------------------------------
# host block manager
# ----------------------------------------------------------------------------
def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class BlockManager:
    """Host block manager (FIFO free list, refcounts, fork, copy-on-write)."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        handle = ctypes.c_void_p()
        order = None if free_order is None else _i32(free_order)
        if order is not None and order.shape != (self.num_blocks,):
            raise ValueError("free_order must list every block once")
        check(lib().pa_bm_create(self.num_blocks, self.block_size, None if order is None else order.ctypes.data,
                                 ctypes.addressof(handle)), "pa_bm_create")
        self.handle = handle.value

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().pa_bm_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    def add_seq(self, seq_id, num_tokens):
        check(lib().pa_bm_add_seq(self.handle, int(seq_id), int(num_tokens)), "pa_bm_add_seq")

    def fork(self, parent, child):
        check(lib().pa_bm_fork(self.handle, int(parent), int(child)), "pa_bm_fork")

    def append_slot(self, seq_id):
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_append_slot(self.handle, int(seq_id), ctypes.addressof(slot), ctypes.addressof(src),
                                      ctypes.addressof(dst)), "pa_bm_append_slot")
        return slot.value, src.value, dst.value

    def step(self, seq_ids, stride=None):
        """Batched append.  Returns (slots, cow_pairs[n_cow][2], tables or None, lens)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        slots = np.empty(n, dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        tables = None if stride is None else np.empty((n, stride), dtype=np.int32)
        n_cow = ctypes.c_int32()
        check(lib().pa_bm_step(self.handle, ids.ctypes.data, n, slots.ctypes.data, pairs.ctypes.data,
                               ctypes.addressof(n_cow), None if tables is None else tables.ctypes.data,
                               0 if stride is None else int(stride), lens.ctypes.data), "pa_bm_step")
        return slots, pairs[:n_cow.value].copy(), tables, lens

    def step_into(self, ids_ptr, n, slots_ptr, pairs_ptr, tables_ptr, stride, lens_ptr):
        """Batched append writing straight into caller buffers (e.g. pinned tensors); returns n_cow."""
        n_cow = ctypes.c_int32()
        check(lib().pa_bm_step(self.handle, ids_ptr, n, slots_ptr, pairs_ptr, ctypes.addressof(n_cow), tables_ptr,
                               stride, lens_ptr), "pa_bm_step")
        return n_cow.value

    def free_seq(self, seq_id):
        check(lib().pa_bm_free_seq(self.handle, int(seq_id)), "pa_bm_free_seq")

    def block_table(self, seq_id):
        nb, nt = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_block_table(self.handle, int(seq_id), None, 0, ctypes.addressof(nb), ctypes.addressof(nt)),
              "pa_bm_block_table")
        out = np.empty(max(nb.value, 1), dtype=np.int32)
        check(lib().pa_bm_block_table(self.handle, int(seq_id), out.ctypes.data, out.shape[0], ctypes.addressof(nb),
                                      ctypes.addressof(nt)), "pa_bm_block_table")
        return out[:nb.value].tolist(), nt.value

    def token_slots(self, seq_id, first=0, count=None):
        if count is None:
            count = self.block_table(seq_id)[1] - first
        out = np.empty(max(count, 1), dtype=np.int32)
        check(lib().pa_bm_token_slots(self.handle, int(seq_id), int(first), int(count), out.ctypes.data),
              "pa_bm_token_slots")
        return out[:count]

    def tables(self, seq_ids, stride):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((ids.shape[0], stride), dtype=np.int32)
        lens = np.empty(ids.shape[0], dtype=np.int32)
        check(lib().pa_bm_tables(self.handle, ids.ctypes.data, ids.shape[0], tables.ctypes.data, int(stride),
                                 lens.ctypes.data), "pa_bm_tables")
        return tables, lens

    def dispatch_order(self, seq_ids):
        """Batch positions in the order to dispatch them (int32 array): long
        sequences first, prefix-sharing sequences side by side."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        order = np.empty(max(ids.shape[0], 1), dtype=np.int32)
        check(lib().pa_bm_dispatch_order(self.handle, ids.ctypes.data, ids.shape[0], order.ctypes.data),
              "pa_bm_dispatch_order")
        return order[:ids.shape[0]]

    def prefix_groups(self, seq_ids):
        """(group_start int32[num_groups + 1], prefix_tokens int32[n],
        max_group_size) of a batch for ``decode_shared_prefix``."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        starts = np.empty(n + 1, dtype=np.int32)
        prefix = np.empty(max(n, 1), dtype=np.int32)
        ng, mg = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_prefix_groups(self.handle, ids.ctypes.data, n, starts.ctypes.data, prefix.ctypes.data,
                                        ctypes.addressof(ng), ctypes.addressof(mg)), "pa_bm_prefix_groups")
        return starts[:ng.value + 1].copy(), prefix[:n].copy(), mg.value

    def prefix_groups_into(self, ids_ptr, n, starts_ptr, prefix_ptr):
        """``prefix_groups`` writing straight into caller buffers (e.g. pinned
        tensors of n + 1 and n int32); returns (num_groups, max_group_size)."""
        ng, mg = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_prefix_groups(self.handle, ids_ptr, n, starts_ptr, prefix_ptr, ctypes.addressof(ng),
                                        ctypes.addressof(mg)), "pa_bm_prefix_groups")
        return ng.value, mg.value

    def _swap(self, seq_id, out):
        n = ctypes.c_int32()
        fn = lib().pa_bm_swap_out if out else lib().pa_bm_swap_in
        name = "pa_bm_swap_out" if out else "pa_bm_swap_in"
        buf = np.empty(1, dtype=np.int32)
        code = fn(self.handle, int(seq_id), buf.ctypes.data, 0, ctypes.addressof(n))
        if code == 0:                      # an empty table: done, no blocks
            return np.empty(0, dtype=np.int32)
        if code != -1:                     # -1: cap 0 was short; n now holds the table length
            check(code, name)
        buf = np.empty(max(n.value, 1), dtype=np.int32)
        check(fn(self.handle, int(seq_id), buf.ctypes.data, buf.shape[0], ctypes.addressof(n)), name)
        return buf[:n.value].copy()

    def swap_out(self, seq_id):
        """Swap a sequence out; returns its blocks in table order (the copy sources)."""
        return self._swap(seq_id, True)

    def swap_in(self, seq_id):
        """Swap a sequence back in; returns its new blocks in table order (the copy destinations)."""
        return self._swap(seq_id, False)

    def refcount(self, block):
        rc = ctypes.c_int32()
        check(lib().pa_bm_refcount(self.handle, int(block), ctypes.addressof(rc)), "pa_bm_refcount")
        return rc.value

    def free_list(self):
        n = ctypes.c_int32()
        check(lib().pa_bm_free_list(self.handle, None, 0, ctypes.addressof(n)), "pa_bm_free_list")
        out = np.empty(max(n.value, 1), dtype=np.int32)
        check(lib().pa_bm_free_list(self.handle, out.ctypes.data, out.shape[0], ctypes.addressof(n)),
              "pa_bm_free_list")
        return out[:n.value].tolist()

    def stats(self):
        st = BmStats()
        check(lib().pa_bm_stats(self.handle, ctypes.addressof(st)), "pa_bm_stats")
        return {name: getattr(st, name) for name, _ in BmStats._fields_}
