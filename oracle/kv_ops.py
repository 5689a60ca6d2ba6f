"""Bitwise KV write and block copy on the paged pool (oracle, test-only).

Pool layout (a reading: the pages require only that each block is contiguous
inside, [P2 §4.2]): one array per tensor, K and V separate, shaped
``[num_blocks][kv_heads][block_size][head_dim]`` and carried as raw bit
patterns (``uint32`` / ``uint16``), so copies are exact byte moves with no float
round-trip.

* ``write_kv`` — decode step 3 of [P2 §3.2.2]: the new token's K and V go to
  the slot its block table assigns.  Slot ``s`` is (block ⌊s/bs⌋, offset
  s mod bs) ([P2 §5]); a slot of -1 means "skip this row" (padding in a
  batch).
* ``swap_out`` / ``swap_in`` — whole blocks to and from a host array shaped
  ``[n][2][kv_heads][block_size][head_dim]`` (block i's K tile, then its V
  tile), the byte moves of swapping ([P2 §5], [P2 §8]).
* ``copy_blocks`` — the copy half of copy-on-write ([P2 §3.4]): the whole
  block (every kv-head, every slot, K and V) is duplicated from src to dst.
  The pairs of one call act as if simultaneous; a call whose destinations
  repeat or overlap any source is rejected, since its result would depend on
  order.
"""
import numpy as np


def write_kv(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Scatter rows of ``k_new``/``v_new`` ([n][kv_heads][head_dim]) into their slots."""
    nb, hkv, bs, d = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("K and V pools differ in shape")
    slots = [int(s) for s in slot_mapping]
    if k_new.shape != (len(slots), hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n][kv_heads][head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != v_pool.dtype:
        raise TypeError("new rows must carry the pool's bit type")
    live = [s for s in slots if s >= 0]
    if len(set(live)) != len(live):
        raise ValueError("two rows target one slot")
    for i, s in enumerate(slots):
        if s < 0:
            continue
        block, offset = divmod(s, bs)
        if block >= nb:
            raise IndexError(f"slot {s} outside the pool")
        k_pool[block, :, offset, :] = k_new[i]
        v_pool[block, :, offset, :] = v_new[i]


def copy_blocks(k_pool, v_pool, pairs):
    """Duplicate whole blocks src → dst for every (src, dst) in ``pairs``."""
    nb = k_pool.shape[0]
    pairs = [(int(a), int(b)) for a, b in pairs]
    srcs = [a for a, _ in pairs]
    dsts = [b for _, b in pairs]
    for b in srcs + dsts:
        if not 0 <= b < nb:
            raise IndexError(f"block {b} outside the pool")
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    if set(dsts) & set(srcs):
        raise ValueError("a destination block is also a source")
    if not pairs:
        return
    k_src = k_pool[srcs].copy()
    v_src = v_pool[srcs].copy()
    k_pool[dsts] = k_src
    v_pool[dsts] = v_src


def swap_out(k_pool, v_pool, blocks):
    """Host copy of whole blocks: out[i][0] = K tile of blocks[i], out[i][1] = its V tile."""
    blocks = [int(b) for b in blocks]
    for b in blocks:
        if not 0 <= b < k_pool.shape[0]:
            raise IndexError(f"block {b} outside the pool")
    return np.stack([k_pool[blocks], v_pool[blocks]], axis=1) if blocks else \
        np.empty((0, 2) + k_pool.shape[1:], dtype=k_pool.dtype)


def swap_in(k_pool, v_pool, blocks, host):
    """Write host[i][0] / host[i][1] into the K / V tile of blocks[i] (distinct blocks)."""
    blocks = [int(b) for b in blocks]
    if len(set(blocks)) != len(blocks):
        raise ValueError("a block is swapped in twice")
    for b in blocks:
        if not 0 <= b < k_pool.shape[0]:
            raise IndexError(f"block {b} outside the pool")
    for i, b in enumerate(blocks):
        k_pool[b] = host[i, 0]
        v_pool[b] = host[i, 1]
