"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (automatic partitioning, outputs in the pool dtype).

State is built by the oracle's block manager from each workload's call
script; the pools are filled on the device by the seeded generator and every
slot that holds no live token is poisoned with NaN.  One decode step is run
through the C ABI: copy-on-write copies (prefix sharing only), the KV write
of the new token, and decode.  Checked against the oracle:

* the whole K and V pools after the step, bit for bit;
* decode outputs of sampled sequences (shortest, longest and seeded picks),
  element by element within 2e-3 (fp16/bf16) / 1e-5 (fp32);
* every output row finite (a NaN would mean a poisoned slot was read).
"""
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from oracle.block_manager import OracleBlockManager
from oracle.kv_ops import write_kv as oracle_write_kv, copy_blocks as oracle_copy_blocks
from workloads import WORKLOADS, make_scenario, device_fill_, seed_for, torch_dtype
from tests.gpu_util import to_bits, out_to_f64, TOL, NAN_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def _apply(ora, ops):
    for op in ops:
        if op[0] == "add":
            ora.add_seq(op[1], op[2])
        elif op[0] == "fork":
            ora.fork(op[1], op[2])
        else:
            ora.step(op[1])


def _fill_and_poison(pool, ora, w, seed):
    """Seeded N(0,1)·scale everywhere, then NaN in every slot no sequence holds."""
    import torch
    device_fill_(pool.k, seed + 1, w.value_scale)
    device_fill_(pool.v, seed + 2, w.value_scale)
    live = np.zeros(pool.num_blocks * w.block_size, dtype=bool)
    for s in ora.seqs:
        live[np.asarray(ora.token_slots(s), dtype=np.int64)] = True
    dead = torch.from_numpy(~live).cuda().view(pool.num_blocks, 1, w.block_size, 1)
    nan = float("nan")
    pool.k.masked_fill_(dead, nan)
    pool.v.masked_fill_(dead, nan)


def _sample(ids, lens, k, seed):
    order = sorted(range(len(ids)), key=lambda i: lens[i])
    picks = {order[0], order[-1]}
    rng = np.random.default_rng(seed)
    while len(picks) < min(k, len(ids)):
        picks.add(int(rng.integers(len(ids))))
    return sorted(picks)


def run_step(pk, name, cow_step=False, samples=16, partition_tokens=None, shared_prefix=False, append=False):
    """One decode step of workload ``name`` on the GPU, checked against the
    oracle (``partition_tokens`` overrides the workload's split).  With
    ``shared_prefix`` the batch is arranged in the oracle's dispatch order and
    decoded by pa_decode_shared_prefix with the oracle's prefix groups; with
    ``append`` the KV write and the decode are one pa_decode_append call."""
    import torch
    w = WORKLOADS[name]
    sc = make_scenario(w)
    seed = seed_for(w)
    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    if cow_step:
        _apply(ora, sc.setup)
        ids = sc.cow_step
    else:
        _apply(ora, sc.all_ops())
        ids = sc.measured
    if shared_prefix:
        ids = [ids[i] for i in ora.dispatch_order(ids)]
    print(f"[{name}{' cow' if cow_step else ''}] {len(ids)} seqs, pool {sc.num_blocks} blocks", flush=True)

    pool = pk.Pool(sc.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype)
    _fill_and_poison(pool, ora, w, seed)
    k_before, v_before = to_bits(pool.k, w.dtype), to_bits(pool.v, w.dtype)

    slots, pairs = ora.step(ids)
    lens = np.array([ora.length(s) for s in ids], dtype=np.int32)
    max_len = int(lens.max())
    stride = -(-max_len // w.block_size)
    tables = np.array(ora.padded_tables(ids, stride, pad=-1), dtype=np.int32)

    tdt = torch_dtype(w.dtype)
    B = len(ids)
    k_new = device_fill_(torch.empty((B, w.kv_heads, w.head_dim), dtype=tdt, device="cuda"), seed + 3, w.value_scale)
    v_new = device_fill_(torch.empty_like(k_new), seed + 4, w.value_scale)
    q = device_fill_(torch.empty((B, w.q_heads, w.head_dim), dtype=tdt, device="cuda"), seed + 5, w.value_scale)

    if pairs:
        pk.copy_blocks(pool, torch.tensor(pairs, dtype=torch.int32, device="cuda"))
    slots_dev = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
    if not append:
        pk.write_kv(pool, k_new, v_new, slots_dev)
    part = w.partition_tokens if partition_tokens is None else partition_tokens
    if shared_prefix:
        starts, prefix, largest = ora.prefix_groups(ids)
        assert max(prefix) > 0
        out = pk.decode_shared_prefix(pool, q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                      max_len, torch.tensor(starts, dtype=torch.int32, device="cuda"),
                                      torch.tensor(prefix, dtype=torch.int32, device="cuda"), largest, max(prefix),
                                      partition_tokens=part)
    else:
        out = pk.decode(pool, q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), max_len,
                        partition_tokens=part, append=(k_new, v_new, slots_dev) if append else None)
    torch.cuda.synchronize()

    # pool bytes after the step: oracle copy + write on the host copy of the start state
    oracle_copy_blocks(k_before, v_before, pairs)
    oracle_write_kv(k_before, v_before, to_bits(k_new, w.dtype), to_bits(v_new, w.dtype), slots)
    assert np.array_equal(to_bits(pool.k, w.dtype), k_before), "K pool differs from the oracle"
    assert np.array_equal(to_bits(pool.v, w.dtype), v_before), "V pool differs from the oracle"

    got = out_to_f64(out)
    assert np.all(np.isfinite(got))
    picks = _sample(ids, lens, samples, seed)
    q_bits = to_bits(q, w.dtype)
    want = paged_decode(q_bits[picks], k_before, v_before, tables[picks], lens[picks], w.dtype)
    err = float(np.max(np.abs(got[picks] - want)))
    print(f"[{name}] sampled seqs {picks}: max |err| = {err:.3e}", flush=True)
    assert err <= TOL[w.dtype]
    return dict(pairs=pairs, lens=lens)


def test_tiny_fp32_full(gpu):
    """The pages' example state: decode before and after the append, everything checked."""
    import torch
    pk = gpu
    w = WORKLOADS["tiny_fp32"]
    sc = make_scenario(w)
    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    _apply(ora, sc.setup)
    rng = np.random.default_rng(seed_for(w))
    k_pool = np.full((16, 1, 4, 64), NAN_BITS["f32"], dtype=np.uint32)
    v_pool = k_pool.copy()
    from tests.gpu_util import draw, to_torch
    pool = pk.Pool(16, 4, 1, 64, "f32", k=to_torch(k_pool, "f32"), v=to_torch(v_pool, "f32"))
    for s in (0, 1):                                   # prefill written through pa_write_kv
        n = ora.length(s)
        kk, vv = draw(rng, (n, 1, 64), "f32", 1.0), draw(rng, (n, 1, 64), "f32", 1.0)
        slots = np.asarray(ora.token_slots(s), dtype=np.int32)
        oracle_write_kv(k_pool, v_pool, kk, vv, slots)
        pk.write_kv(pool, to_torch(kk, "f32"), to_torch(vv, "f32"), torch.from_numpy(slots).cuda())
    q = draw(rng, (2, 1, 64), "f32", 1.0)
    tables = np.array(ora.padded_tables([0, 1], 3, pad=-1), dtype=np.int32)
    assert tables.tolist() == [[5, 12, 3], [9, 0, -1]]
    lens = np.array([10, 7], dtype=np.int32)
    out = pk.decode(pool, to_torch(q, "f32"), torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), 10)
    want = paged_decode(q, k_pool, v_pool, tables, lens, "f32")
    assert np.max(np.abs(out_to_f64(out) - want)) <= TOL["f32"]
    # the step: append one token each, write, decode over 11 and 8 tokens
    slots, pairs = ora.step([0, 1])
    assert slots == [14, 3] and pairs == []
    kn, vn = draw(rng, (2, 1, 64), "f32", 1.0), draw(rng, (2, 1, 64), "f32", 1.0)
    oracle_write_kv(k_pool, v_pool, kn, vn, slots)
    pk.write_kv(pool, to_torch(kn, "f32"), to_torch(vn, "f32"), torch.tensor(slots, dtype=torch.int32).cuda())
    tables = np.array(ora.padded_tables([0, 1], 3, pad=-1), dtype=np.int32)
    lens = np.array([11, 8], dtype=np.int32)
    out = pk.decode(pool, to_torch(q, "f32"), torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), 11)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(pool.k, "f32"), k_pool) and np.array_equal(to_bits(pool.v, "f32"), v_pool)
    want = paged_decode(q, k_pool, v_pool, tables, lens, "f32")
    assert np.max(np.abs(out_to_f64(out) - want)) <= TOL["f32"]


def test_mha7b_fp16_full(gpu):
    run_step(gpu, "mha7b_fp16")


def test_gqa70b_bf16_full(gpu):
    run_step(gpu, "gqa70b_bf16")


@pytest.mark.parametrize("partition", [512, -1, -2])
def test_gqa70b_bf16_split_full(gpu, partition):
    """The GQA batch split into 512-token partitions (16384 rows for the
    reduce kernel, one workgroup per row), by the balanced split and by the
    uniform split (2048 units: one workgroup each, no reduce)."""
    run_step(gpu, "gqa70b_bf16", partition_tokens=partition)


def test_prefix_share_cow_step_full(gpu):
    r = run_step(gpu, "prefix_share_fp16", cow_step=True, samples=16)
    assert len(r["pairs"]) == 224


def test_prefix_share_steady_full(gpu):
    r = run_step(gpu, "prefix_share_fp16")
    assert r["pairs"] == []


@pytest.mark.parametrize("cow_step", [False, True])
def test_prefix_share_shared_prefix_decode_full(gpu, cow_step):
    """The prefix-sharing batch (32 prompts x 8 samples) through the
    sharing-aware decode: each prompt's 1024-token prefix read once per
    kv-head, checked on sampled sequences against the oracle."""
    r = run_step(gpu, "prefix_share_fp16", cow_step=cow_step, samples=16, shared_prefix=True)
    assert len(r["pairs"]) == (224 if cow_step else 0)


@pytest.mark.parametrize("partition", [None, -2])
def test_long_splitk_bf16_full(gpu, partition):
    """The long-context batch with the workload's 512-token partitions and
    with the uniform split (~1100-token partitions, one resident grid)."""
    run_step(gpu, "long_splitk_bf16", samples=8, partition_tokens=partition)


@pytest.mark.parametrize("name,partition,cow_step", [
    ("mha7b_fp16", None, False),
    ("gqa70b_bf16", None, False),
    ("gqa70b_bf16", 512, False),
    ("gqa70b_bf16", -2, False),
    ("gqa70b_bf16", -1, False),
    ("prefix_share_fp16", None, True),
    ("long_splitk_bf16", None, False),
    ("long_splitk_bf16", -2, False),
])
def test_decode_append_full(gpu, name, partition, cow_step):
    """The step as pa_decode_append (KV write inside the decode launch): whole
    sequences, fixed partitions, the uniform split, and the balanced split
    (where the library writes first); the pool is checked bit for bit and the
    outputs against the oracle, as for the two-call step."""
    run_step(gpu, name, cow_step=cow_step, samples=4, partition_tokens=partition, append=True)
