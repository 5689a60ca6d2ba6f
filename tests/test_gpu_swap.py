"""GPU parity of block swap (pa_swap_out / pa_swap_in) against the oracle.

The oracle block manager decides which blocks leave and which come back; the
bytes that reach pinned host memory must equal the oracle's tiles bit for
bit, the pool after swap-in must equal the oracle's pool bit for bit (the
blocks freed by swap-out are poisoned first, as a later writer would), and a
decode through the new table must match the fp64 oracle.
"""
import ctypes
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from oracle.kv_ops import swap_out as oracle_swap_out, swap_in as oracle_swap_in
from tests.gpu_util import build_case, to_torch, to_bits, out_to_f64, TOL, NAN_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


@pytest.mark.parametrize("dtype,kv_heads,head_dim,bs", [("f16", 2, 128, 16), ("bf16", 1, 64, 32),
                                                        ("f32", 2, 64, 4)])
def test_swap_round_trip_bit_exact(gpu, dtype, kv_heads, head_dim, bs):
    import torch
    pk = gpu
    lens = [37, 5, 64, 0, 100]
    case = build_case(lens, kv_heads, 2, head_dim, bs, dtype, seed=31 + bs)
    bm, kp, vp = case["bm"], case["k_pool"], case["v_pool"]
    pool = pk.Pool(case["num_blocks"], bs, kv_heads, head_dim, dtype, k=to_torch(kp, dtype), v=to_torch(vp, dtype))
    for victim in (4, 2):
        blocks = bm.swap_out(victim)
        host = torch.empty(len(blocks) * 2 * pool.block_bytes, dtype=torch.uint8, pin_memory=True)
        pk.swap_out(pool, torch.tensor(blocks, dtype=torch.int32, device="cuda"), host)
        torch.cuda.synchronize()
        want = oracle_swap_out(kp, vp, blocks)
        assert host.numpy().tobytes() == want.tobytes()
        # the released blocks are free for others: poison them everywhere
        idx = torch.tensor(blocks, dtype=torch.long, device="cuda")
        pool.k[idx] = float("nan")
        pool.v[idx] = float("nan")
        kp[blocks] = NAN_BITS[dtype]
        vp[blocks] = NAN_BITS[dtype]
        new = bm.swap_in(victim)
        pk.swap_in(pool, torch.tensor(new, dtype=torch.int32, device="cuda"), host)
        oracle_swap_in(kp, vp, new, want)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(pool.k, dtype), kp) and np.array_equal(to_bits(pool.v, dtype), vp)
    stride = max(-(-n // bs) for n in lens)
    tables = np.array(bm.padded_tables(range(len(lens)), stride, pad=-1), dtype=np.int32)
    q = to_torch(case["q"], dtype)
    out = pk.decode(pool, q, torch.from_numpy(tables).cuda(), torch.from_numpy(case["lens"]).cuda(), max(lens),
                    out_dtype="f32")
    want = paged_decode(case["q"], kp, vp, tables, case["lens"], dtype)
    assert np.max(np.abs(out_to_f64(out) - want)) <= TOL[dtype]


def test_swap_rejects_memory_it_cannot_map(gpu):
    import torch
    pk = gpu
    from paged_kv_cache_355_amd._lib import lib
    case = build_case([20], 1, 1, 64, 16, "f16", seed=5)
    pool = pk.Pool(case["num_blocks"], 16, 1, 64, "f16", k=to_torch(case["k_pool"], "f16"),
                   v=to_torch(case["v_pool"], "f16"))
    blocks = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        pk.swap_out(pool, blocks, torch.empty(2 * 2 * pool.block_bytes, dtype=torch.uint8))   # not pinned
    pageable = np.zeros(2 * 2 * pool.block_bytes, dtype=np.uint8)
    code = lib().pa_swap_out(pool.handle, blocks.data_ptr(), 2, pageable.ctypes.data, pageable.nbytes, None)
    assert code == -1                                                   # PA_ERR_INVALID, nothing launched
    small = torch.empty(2 * pool.block_bytes, dtype=torch.uint8, pin_memory=True)
    with pytest.raises(pk.PaError):
        pk.swap_out(pool, blocks, small)                               # room for one block, not two
    host = torch.empty(2 * 2 * pool.block_bytes, dtype=torch.uint8, pin_memory=True)
    with pytest.raises(pk.PaError):
        pk.swap_in(pool, torch.tensor([3, 3], dtype=torch.int32, device="cuda"), host)   # twice (validation)
    assert not np.any(pageable)
