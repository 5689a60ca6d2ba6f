"""Helpers for the GPU parity tests: moving stored bit patterns between numpy
and torch, and building small paged cases through the oracle's block manager.

Inputs come from the seeded generators (workloads) and the oracle; nothing
here computes what the library computes.
"""
import math

import numpy as np

from oracle.block_manager import OracleBlockManager
from oracle.kv_ops import write_kv as oracle_write_kv
from workloads import round_to_bits

NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def to_torch(bits, dtype, device="cuda"):
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).view(torch.float32)
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to(device)


def to_bits(t, dtype):
    import torch
    if dtype == "f32":
        return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def out_to_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def draw(rng, shape, dtype, scale):
    return round_to_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale), dtype)


def build_case(lengths, kv_heads, group, head_dim, block_size, dtype, seed, scale=1.0, extra_blocks=3):
    """Random K/V for each sequence written through the oracle into a NaN-poisoned pool."""
    rng = np.random.default_rng(seed)
    bs = block_size
    nb = sum(-(-n // bs) for n in lengths) + extra_blocks
    order = rng.permutation(nb)
    bm = OracleBlockManager(nb, bs, order)
    bits_t = np.uint32 if dtype == "f32" else np.uint16
    shape = (nb, kv_heads, bs, head_dim)
    k_pool = np.full(shape, NAN_BITS[dtype], dtype=bits_t)
    v_pool = k_pool.copy()
    for s, n in enumerate(lengths):
        bm.add_seq(s, n)
        oracle_write_kv(k_pool, v_pool, draw(rng, (n, kv_heads, head_dim), dtype, scale),
                        draw(rng, (n, kv_heads, head_dim), dtype, scale), bm.token_slots(s))
    q = draw(rng, (len(lengths), kv_heads * group, head_dim), dtype, scale)
    stride = max([-(-n // bs) for n in lengths] + [1])
    tables = np.array(bm.padded_tables(range(len(lengths)), stride, pad=-1), dtype=np.int32)
    return dict(bm=bm, k_pool=k_pool, v_pool=v_pool, q=q, tables=tables,
                lens=np.array(lengths, dtype=np.int32), num_blocks=nb)


def run_decode(pk, case, kv_heads, head_dim, block_size, dtype, out_dtype=None, partition_tokens=0,
               k_pool=None, v_pool=None):
    import torch
    k = to_torch(case["k_pool"] if k_pool is None else k_pool, dtype)
    v = to_torch(case["v_pool"] if v_pool is None else v_pool, dtype)
    pool = pk.Pool(case["num_blocks"], block_size, kv_heads, head_dim, dtype, k=k, v=v)
    q = to_torch(case["q"], dtype)
    tables = torch.from_numpy(case["tables"]).cuda()
    lens = torch.from_numpy(case["lens"]).cuda()
    out = pk.decode(pool, q, tables, lens, int(max(case["lens"].max(), 0)), out_dtype=out_dtype,
                    partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


def peak_key(case, seq, token, kv_head, group_rows, logit, head_dim, dtype, block_size):
    """Make key ``token`` of ``seq``/``kv_head`` a multiple of the first query row of the group,
    so its scaled logit for that row is ``logit``; returns nothing, edits case in place."""
    from oracle.numerics import to_f64
    q_row = to_f64(case["q"][seq, kv_head * group_rows], dtype)
    denom = float(q_row @ q_row) / math.sqrt(head_dim)
    alpha = logit / denom
    kf = round_to_bits((q_row * alpha).astype(np.float32), dtype)
    table = case["tables"][seq]
    b = int(table[token // block_size])
    case["k_pool"][b, kv_head, token % block_size, :] = kf


def build_families(families, kv_heads, group, head_dim, block_size, dtype, seed, scale=1.0, extra_blocks=4):
    """Fork families written through the oracle into a NaN-poisoned pool.

    ``families`` lists (prompt_len, [appended tokens per member]): member 0 is
    the prompt's own sequence, the others fork from it before any append, and
    each member then appends its tokens one at a time (copy-on-write copies
    applied to the pool as the oracle block manager emits them).  The batch
    is arranged by the oracle's dispatch order; returns the case dict of
    ``build_case`` plus ``ids``, ``group_start``, ``prefix`` and
    ``max_group``, the oracle's prefix groups of that batch."""
    from oracle.kv_ops import copy_blocks as oracle_copy_blocks
    rng = np.random.default_rng(seed)
    bs = block_size
    need = sum(-(-(p + max(app) + 1) // bs) * len(app) for p, app in families) + extra_blocks
    order = rng.permutation(need)
    bm = OracleBlockManager(need, bs, order)
    bits_t = np.uint32 if dtype == "f32" else np.uint16
    shape = (need, kv_heads, bs, head_dim)
    k_pool = np.full(shape, NAN_BITS[dtype], dtype=bits_t)
    v_pool = k_pool.copy()
    ids = []
    for f, (prompt, appends) in enumerate(families):
        root = (f, 0)
        bm.add_seq(root, prompt)
        oracle_write_kv(k_pool, v_pool, draw(rng, (prompt, kv_heads, head_dim), dtype, scale),
                        draw(rng, (prompt, kv_heads, head_dim), dtype, scale), bm.token_slots(root))
        members = [root]
        for c in range(1, len(appends)):
            bm.fork(root, (f, c))
            members.append((f, c))
        for m, n in zip(members, appends):
            for _ in range(n):
                slot, src, dst = bm.append_slot(m)
                if src >= 0:
                    oracle_copy_blocks(k_pool, v_pool, [(src, dst)])
                oracle_write_kv(k_pool, v_pool, draw(rng, (1, kv_heads, head_dim), dtype, scale),
                                draw(rng, (1, kv_heads, head_dim), dtype, scale), [slot])
        ids.extend(members)
    ids = [ids[i] for i in bm.dispatch_order(ids)]
    lens = np.array([bm.length(s) for s in ids], dtype=np.int32)
    stride = max([-(-int(n) // bs) for n in lens] + [1])
    tables = np.array(bm.padded_tables(ids, stride, pad=-1), dtype=np.int32)
    q = draw(rng, (len(ids), kv_heads * group, head_dim), dtype, scale)
    starts, prefix, largest = bm.prefix_groups(ids)
    return dict(bm=bm, k_pool=k_pool, v_pool=v_pool, q=q, tables=tables, lens=lens, num_blocks=need, ids=ids,
                group_start=np.array(starts, dtype=np.int32), prefix=np.array(prefix, dtype=np.int32),
                max_group=largest)


def run_shared_prefix(pk, case, kv_heads, head_dim, block_size, dtype, out_dtype=None, partition_tokens=0,
                      group_start=None, prefix=None, max_prefix=None):
    import torch
    k = to_torch(case["k_pool"], dtype)
    v = to_torch(case["v_pool"], dtype)
    pool = pk.Pool(case["num_blocks"], block_size, kv_heads, head_dim, dtype, k=k, v=v)
    gs = case["group_start"] if group_start is None else group_start
    pre = case["prefix"] if prefix is None else prefix
    max_len = int(max(case["lens"].max(), 0))
    out = pk.decode_shared_prefix(
        pool, to_torch(case["q"], dtype), torch.from_numpy(case["tables"]).cuda(),
        torch.from_numpy(case["lens"]).cuda(), max_len, torch.from_numpy(np.asarray(gs, dtype=np.int32)).cuda(),
        torch.from_numpy(np.asarray(pre, dtype=np.int32)).cuda(), case["max_group"],
        int(pre.max()) if max_prefix is None else max_prefix, out_dtype=out_dtype,
        partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out
