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
