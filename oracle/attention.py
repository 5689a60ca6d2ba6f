"""Paged single-query decode attention in float64 (oracle, test-only).

What it computes is the plain definition, since paging only moves where K/V
live and tiled or split softmax only regroups a sum:

* [P2 §1.1]: attention is softmax(q Kᵀ / √d) V.  Decode has one query row per
  head and the keys/values of every cached token of the sequence ([P2 §3.2.2]
  step 4: all logical blocks of the table are visited).
* [P2 §2.3], [P2 §5], [P1 "块表（Block Table）"]: token t of a sequence is
  found through its block table — physical block ``table[⌊t/bs⌋]``, offset
  ``t mod bs``.

So, for each sequence, this module first rebuilds the sequence's contiguous
K and V from its block table, widened exactly to float64, and then evaluates
the formula head by head.

Readings (the pages are silent on these):

* Grouped-query attention: query head h reads kv-head ⌊h / G⌋ with
  G = q_heads / kv_heads, so consecutive query heads share a kv-head.
* The scale defaults to 1/√head_dim; a caller may override it.
* A context length of 0 yields an all-zero output row.
* Slots past the context length (the last block's padding, [P2 §3.2.1]) hold
  undefined values and are never read.
"""
import numpy as np

from .numerics import to_f64


def gather_sequence(pool, table, length, block_size):
    """Contiguous ``[kv_heads][length][head_dim]`` copy of one sequence's tokens.

    ``pool`` is ``[num_blocks][kv_heads][block_size][head_dim]`` (stored bits
    or floats; the element type is kept); tokens are visited in logical order
    and each is fetched through the table.
    """
    nb, hkv, bs, d = pool.shape
    assert bs == block_size
    out = np.empty((hkv, length, d), dtype=pool.dtype)
    for t in range(length):
        block = int(table[t // block_size])
        if not 0 <= block < nb:
            raise IndexError(f"table entry {block} outside the pool")
        out[:, t, :] = pool[block, :, t % block_size, :]
    return out


def softmax_attend(q, keys, values, scale):
    """softmax(keys·q·scale) · values for one query row (all float64)."""
    logits = (keys @ q) * scale
    logits = logits - logits.max()
    weights = np.exp(logits)
    weights = weights / weights.sum()
    return weights @ values


def paged_decode(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
                 dtype, scale=None, q_dtype=None):
    """Decode attention for a batch.

    q_bits:        [B][q_heads][head_dim] stored bits of the queries
    k/v_pool_bits: [num_blocks][kv_heads][block_size][head_dim] stored bits
    block_tables:  B rows of physical block ids (entries past ⌈len/bs⌉ unused)
    context_lens:  [B] tokens to attend over (0 → zero output)
    Returns float64 [B][q_heads][head_dim].
    """
    q_dtype = dtype if q_dtype is None else q_dtype
    nb, hkv, bs, d = k_pool_bits.shape
    B, hq, dq = q_bits.shape
    if dq != d or hq % hkv != 0:
        raise ValueError("q must be [B][q_heads][head_dim] with q_heads a multiple of kv_heads")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = to_f64(q_bits, q_dtype)
    out = np.zeros((B, hq, d), dtype=np.float64)
    for s in range(B):
        length = int(context_lens[s])
        if length == 0:
            continue
        k_seq = to_f64(gather_sequence(k_pool_bits, block_tables[s], length, bs), dtype)
        v_seq = to_f64(gather_sequence(v_pool_bits, block_tables[s], length, bs), dtype)
        for h in range(hq):
            g = h // group
            out[s, h] = softmax_attend(qf[s, h], k_seq[g], v_seq[g], scale)
    return out

