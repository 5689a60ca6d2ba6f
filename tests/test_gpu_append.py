"""pa_decode_append: the step's KV write and the decode in one launch
([P2] §3.2.2 steps 3 and 4).

Each case holds every token of every sequence; the last token of most
sequences is then taken out of the pool (its slot poisoned with NaN) and
handed to pa_decode_append as the new token.  Checked:

* the pool after the call equals the pool with every token written, bit for bit;
* the output equals pa_decode's on that full pool bit for bit (the same
  kernels read the same bytes), and the fp64 oracle within tolerance;
* slots of -1 (token already in the pool), empty sequences and every split
  mode, including the balanced split, where the library writes first.
"""
import os

import numpy as np
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_case, to_torch, to_bits, out_to_f64, NAN_BITS, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def _case(dtype, head_dim, block_size, group, kv_heads, lengths, seed):
    case = build_case(lengths, kv_heads, group, head_dim, block_size, dtype, seed, scale=head_dim ** -0.5)
    bm = case["bm"]
    rng = np.random.default_rng(seed + 7)
    B = len(lengths)
    bits_t = case["k_pool"].dtype
    k_new = np.zeros((B, kv_heads, head_dim), dtype=bits_t)
    v_new = np.zeros_like(k_new)
    slots = np.full(B, -1, dtype=np.int32)
    k_gap, v_gap = case["k_pool"].copy(), case["v_pool"].copy()
    for s, n in enumerate(lengths):
        if n == 0 or rng.random() < 0.2:   # nothing new for this sequence: slot -1
            continue
        slot = bm.token_slots(s)[n - 1]
        b, o = divmod(slot, block_size)
        slots[s] = slot
        k_new[s], v_new[s] = case["k_pool"][b, :, o, :], case["v_pool"][b, :, o, :]
        k_gap[b, :, o, :] = NAN_BITS[dtype]
        v_gap[b, :, o, :] = NAN_BITS[dtype]
    return case, k_new, v_new, slots, k_gap, v_gap


def _lengths(block_size, rng):
    ls = [0, 1, block_size - 1, block_size, block_size + 1, 3 * block_size + 5, 40 * block_size + 3]
    ls += [int(x) for x in rng.integers(1, 30 * block_size, size=9)]
    return ls


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("head_dim,block_size", [(64, 4), (128, 16), (128, 32), (64, 64)])
@pytest.mark.parametrize("group", [1, 8])
@pytest.mark.parametrize("partition", [0, 64, -1, -2])
def test_append_equals_write_then_decode(gpu, dtype, head_dim, block_size, group, partition):
    import torch
    pk = gpu
    kv_heads = 2
    seed = 9000 + head_dim + block_size + group + (partition & 0xFF)
    lengths = _lengths(block_size, np.random.default_rng(seed))
    part = partition if partition <= 0 else max(partition // block_size, 1) * block_size
    print(f"[append] {dtype} d{head_dim} bs{block_size} G{group} partition {part}", flush=True)
    case, k_new, v_new, slots, k_gap, v_gap = _case(dtype, head_dim, block_size, group, kv_heads, lengths, seed)
    tables = torch.from_numpy(case["tables"]).cuda()
    lens = torch.from_numpy(case["lens"]).cuda()
    q = to_torch(case["q"], dtype)
    max_len = int(case["lens"].max())

    full = pk.Pool(case["num_blocks"], block_size, kv_heads, head_dim, dtype,
                   k=to_torch(case["k_pool"], dtype), v=to_torch(case["v_pool"], dtype))
    want = pk.decode(full, q, tables, lens, max_len, partition_tokens=part)

    gap = pk.Pool(case["num_blocks"], block_size, kv_heads, head_dim, dtype,
                  k=to_torch(k_gap, dtype), v=to_torch(v_gap, dtype))
    got = pk.decode(gap, q, tables, lens, max_len, partition_tokens=part,
                    append=(to_torch(k_new, dtype), to_torch(v_new, dtype), torch.from_numpy(slots).cuda()))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(gap.k, dtype), case["k_pool"]), "K pool after the append differs"
    assert np.array_equal(to_bits(gap.v, dtype), case["v_pool"]), "V pool after the append differs"
    assert np.array_equal(to_bits(got, dtype), to_bits(want, dtype)), "output differs from write + decode"
    ref = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], dtype)
    assert np.max(np.abs(out_to_f64(got) - ref)) <= TOL[dtype]


def test_append_rejects_a_slot_that_is_not_the_last_token(gpu):
    import torch
    pk = gpu
    case, k_new, v_new, slots, k_gap, v_gap = _case("f16", 128, 16, 1, 2, [20, 33, 5], 77)
    bad = slots.copy()
    bad[0] = case["bm"].token_slots(0)[0]   # sequence 0's first token's slot instead of its last's
    pool = pk.Pool(case["num_blocks"], 16, 2, 128, "f16", k=to_torch(k_gap, "f16"), v=to_torch(v_gap, "f16"))
    with pytest.raises(pk.PaError, match="context_lens - 1"):
        pk.decode(pool, to_torch(case["q"], "f16"), torch.from_numpy(case["tables"]).cuda(),
                  torch.from_numpy(case["lens"]).cuda(), 33,
                  append=(to_torch(k_new, "f16"), to_torch(v_new, "f16"), torch.from_numpy(bad).cuda()))
