"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (automatic partitioning, outputs in the pool dtype), driven
by the library's own block manager.

Each workload's call script builds the same state twice: in the library's
block manager (pa_bm_* through the C ABI) and in the oracle's.  The batch is
arranged by the library's dispatch order and stepped by pa_bm_step into
block tables padded with -1 past each table (a stride longer than needed);
its slots, copy-on-write pairs, tables, lengths, order and (for the
sharing-aware decode) prefix groups must equal the oracle's, and they are
what the kernels run on.  The pools are filled on the device by the seeded
generator and every slot that holds no live token is poisoned with NaN.  The
step then runs through the C ABI: copy-on-write copies, the KV write of the
new token, decode.  Checked against the oracle:

* the whole K and V pools after the step, bit for bit;
* EVERY output row of the batch, element by element, within 2e-3
  (fp16/bf16) / 1e-5 (fp32) of the fp64 oracle.

The oracle's result depends only on the state, not on how the library splits
the work, so it is computed once per state and reused by the split-mode and
fused-append variants of the same step.
"""
import math
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from oracle.block_manager import OracleBlockManager
from oracle.numerics import to_f64
from oracle.kv_ops import write_kv as oracle_write_kv, copy_blocks as oracle_copy_blocks
from workloads import WORKLOADS, make_scenario, device_fill_, seed_for, torch_dtype, round_to_bits
from tests.gpu_util import to_bits, to_torch, out_to_f64, TOL, NAN_BITS

pytestmark = pytest.mark.gpu

# expected decode rows per (workload, step kind, value scale): q bits, tables, lengths, oracle output
_EXPECTED = {}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def _apply(mgr, ops):
    """Run a workload's call script on either block manager."""
    for op in ops:
        if op[0] == "add":
            mgr.add_seq(op[1], op[2])
        elif op[0] == "fork":
            mgr.fork(op[1], op[2])
        else:
            mgr.step(op[1])


def _fill_and_poison(pool, ora, w, seed, scale):
    """Seeded N(0,1)·scale everywhere, then NaN in every slot no sequence holds."""
    import torch
    device_fill_(pool.k, seed + 1, scale)
    device_fill_(pool.v, seed + 2, scale)
    live = np.zeros(pool.num_blocks * w.block_size, dtype=bool)
    for s in ora.seqs:
        live[np.asarray(ora.token_slots(s), dtype=np.int64)] = True
    dead = torch.from_numpy(~live).cuda().view(pool.num_blocks, 1, w.block_size, 1)
    nan = float("nan")
    pool.k.masked_fill_(dead, nan)
    pool.v.masked_fill_(dead, nan)


def library_step_state(pk, name, cow_step=False, stride_pad=3):
    """The workload's state in both block managers, the batch in the library's
    dispatch order (checked against the oracle's), and a pool filled and
    poisoned for it.  Returns a dict; the step itself is not taken yet."""
    w = WORKLOADS[name]
    sc = make_scenario(w)
    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    bm = pk.BlockManager(sc.num_blocks, w.block_size, sc.free_order)
    ops = sc.setup if cow_step else sc.all_ops()
    _apply(ora, ops)
    _apply(bm, ops)
    ids = list(sc.cow_step if cow_step else sc.measured)
    order = bm.dispatch_order(ids)
    assert order.tolist() == ora.dispatch_order(ids), "dispatch order differs from the oracle's"
    ids = [ids[i] for i in order]
    stride = -(-(max(ora.length(s) for s in ids) + 1) // w.block_size) + stride_pad
    return dict(w=w, sc=sc, ora=ora, bm=bm, ids=ids, stride=stride, seed=seed_for(w))


def library_step(st, shared_prefix=False):
    """pa_bm_step (and pa_bm_prefix_groups) on the library's manager; every
    output is checked against the oracle's own step.  Returns the library's
    arrays."""
    bm, ora, ids, stride = st["bm"], st["ora"], st["ids"], st["stride"]
    slots, pairs, tables, lens = bm.step(ids, stride=stride)
    o_slots, o_pairs = ora.step(ids)
    assert slots.tolist() == o_slots, "slot mapping differs from the oracle's"
    assert [tuple(p) for p in pairs.tolist()] == [tuple(p) for p in o_pairs], "copy-on-write pairs differ"
    assert tables.tolist() == ora.padded_tables(ids, stride, pad=-1), "padded block tables differ"
    assert lens.tolist() == [ora.length(s) for s in ids], "context lengths differ"
    res = dict(slots=slots, pairs=pairs, tables=tables, lens=lens, o_slots=o_slots, o_pairs=o_pairs)
    if shared_prefix:
        starts, prefix, largest = bm.prefix_groups(ids)
        o_starts, o_prefix, o_largest = ora.prefix_groups(ids)
        assert starts.tolist() == o_starts and prefix.tolist() == o_prefix and largest == o_largest, \
            "prefix groups differ from the oracle's"
        assert max(o_prefix) > 0
        res.update(starts=starts, prefix=prefix, largest=largest)
    return res


def expected_rows(key, q_bits, k_pool, v_pool, tables, lens, dtype):
    """Oracle output of every row, computed once per state key."""
    hit = _EXPECTED.get(key)
    if hit is not None:
        q0, t0, l0, want = hit
        if np.array_equal(q0, q_bits) and np.array_equal(t0, tables) and np.array_equal(l0, lens):
            return want
    want = paged_decode(q_bits, k_pool, v_pool, tables, lens, dtype)
    _EXPECTED[key] = (q_bits.copy(), tables.copy(), lens.copy(), want)
    return want


def run_step(pk, name, cow_step=False, partition_tokens=None, shared_prefix=False, append=False):
    """One decode step of workload ``name`` on the GPU from the library's block
    manager, checked against the oracle (``partition_tokens`` overrides the
    workload's split).  With ``shared_prefix`` the step decodes through
    pa_decode_shared_prefix with the library's prefix groups; with ``append``
    the KV write and the decode are one pa_decode_append call."""
    import torch
    st = library_step_state(pk, name, cow_step)
    w, ora, ids, seed = st["w"], st["ora"], st["ids"], st["seed"]
    print(f"[{name}{' cow' if cow_step else ''}] {len(ids)} seqs, pool {st['sc'].num_blocks} blocks, "
          f"split {partition_tokens}, shared_prefix {shared_prefix}, append {append}", flush=True)

    pool = pk.Pool(st["sc"].num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype)
    _fill_and_poison(pool, ora, w, seed, w.value_scale)
    k_before, v_before = to_bits(pool.k, w.dtype), to_bits(pool.v, w.dtype)
    step = library_step(st, shared_prefix)
    lens, tables = step["lens"], step["tables"]
    max_len = int(lens.max())

    tdt = torch_dtype(w.dtype)
    B = len(ids)
    k_new = device_fill_(torch.empty((B, w.kv_heads, w.head_dim), dtype=tdt, device="cuda"), seed + 3, w.value_scale)
    v_new = device_fill_(torch.empty_like(k_new), seed + 4, w.value_scale)
    q = device_fill_(torch.empty((B, w.q_heads, w.head_dim), dtype=tdt, device="cuda"), seed + 5, w.value_scale)

    if step["pairs"].shape[0]:
        pk.copy_blocks(pool, torch.from_numpy(np.ascontiguousarray(step["pairs"])).cuda())
    slots_dev = torch.from_numpy(step["slots"]).cuda()
    if not append:
        pk.write_kv(pool, k_new, v_new, slots_dev)
    part = w.partition_tokens if partition_tokens is None else partition_tokens
    tables_dev, lens_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    if shared_prefix:
        out = pk.decode_shared_prefix(pool, q, tables_dev, lens_dev, max_len, torch.from_numpy(step["starts"]).cuda(),
                                      torch.from_numpy(step["prefix"]).cuda(), step["largest"],
                                      int(step["prefix"].max()), partition_tokens=part)
    else:
        out = pk.decode(pool, q, tables_dev, lens_dev, max_len, partition_tokens=part,
                        append=(k_new, v_new, slots_dev) if append else None)
    torch.cuda.synchronize()

    # pool bytes after the step: the oracle's copy + write on the host copy of the start state
    oracle_copy_blocks(k_before, v_before, step["o_pairs"])
    oracle_write_kv(k_before, v_before, to_bits(k_new, w.dtype), to_bits(v_new, w.dtype), step["o_slots"])
    assert np.array_equal(to_bits(pool.k, w.dtype), k_before), "K pool differs from the oracle"
    assert np.array_equal(to_bits(pool.v, w.dtype), v_before), "V pool differs from the oracle"

    got = out_to_f64(out)
    o_tables = np.array(ora.padded_tables(ids, st["stride"], pad=-1), dtype=np.int32)
    want = expected_rows((name, cow_step, w.value_scale), to_bits(q, w.dtype), k_before, v_before, o_tables,
                         lens.copy(), w.dtype)
    err = np.abs(got - want).reshape(B, -1).max(axis=1)
    worst = int(np.argmax(err))
    print(f"[{name}] all {B} rows: max |err| = {err[worst]:.3e} (position {worst})", flush=True)
    assert err[worst] <= TOL[w.dtype], f"row {worst} differs by {err[worst]:.3e}"
    return dict(pairs=step["o_pairs"], lens=lens)


def test_tiny_fp32_full(gpu):
    """The pages' example state: decode before and after the append, everything checked."""
    import torch
    pk = gpu
    w = WORKLOADS["tiny_fp32"]
    sc = make_scenario(w)
    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    bm = pk.BlockManager(sc.num_blocks, w.block_size, sc.free_order)
    _apply(ora, sc.setup)
    _apply(bm, sc.setup)
    rng = np.random.default_rng(seed_for(w))
    k_pool = np.full((16, 1, 4, 64), NAN_BITS["f32"], dtype=np.uint32)
    v_pool = k_pool.copy()
    from tests.gpu_util import draw
    pool = pk.Pool(16, 4, 1, 64, "f32", k=to_torch(k_pool, "f32"), v=to_torch(v_pool, "f32"))
    for s in (0, 1):                                   # prefill written through pa_write_kv
        n = ora.length(s)
        kk, vv = draw(rng, (n, 1, 64), "f32", 1.0), draw(rng, (n, 1, 64), "f32", 1.0)
        slots = bm.token_slots(s)
        assert slots.tolist() == ora.token_slots(s)
        oracle_write_kv(k_pool, v_pool, kk, vv, slots)
        pk.write_kv(pool, to_torch(kk, "f32"), to_torch(vv, "f32"), torch.from_numpy(slots).cuda())
    q = draw(rng, (2, 1, 64), "f32", 1.0)
    tables, lens = bm.tables([0, 1], 3)
    assert tables.tolist() == [[5, 12, 3], [9, 0, -1]] == ora.padded_tables([0, 1], 3, pad=-1)
    assert lens.tolist() == [10, 7]
    out = pk.decode(pool, to_torch(q, "f32"), torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), 10)
    want = paged_decode(q, k_pool, v_pool, tables, lens, "f32")
    assert np.max(np.abs(out_to_f64(out) - want)) <= TOL["f32"]
    # the step: append one token each, write, decode over 11 and 8 tokens
    slots, pairs, tables, lens = bm.step([0, 1], stride=3)
    o_slots, o_pairs = ora.step([0, 1])
    assert slots.tolist() == o_slots == [14, 3] and pairs.shape[0] == 0 and o_pairs == []
    kn, vn = draw(rng, (2, 1, 64), "f32", 1.0), draw(rng, (2, 1, 64), "f32", 1.0)
    oracle_write_kv(k_pool, v_pool, kn, vn, o_slots)
    pk.write_kv(pool, to_torch(kn, "f32"), to_torch(vn, "f32"), torch.from_numpy(slots).cuda())
    assert tables.tolist() == ora.padded_tables([0, 1], 3, pad=-1) and lens.tolist() == [11, 8]
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
    r = run_step(gpu, "prefix_share_fp16", cow_step=True)
    assert len(r["pairs"]) == 224


def test_prefix_share_steady_full(gpu):
    r = run_step(gpu, "prefix_share_fp16")
    assert r["pairs"] == []


@pytest.mark.parametrize("cow_step", [False, True])
def test_prefix_share_shared_prefix_decode_full(gpu, cow_step):
    """The prefix-sharing batch (32 prompts x 8 samples) through the
    sharing-aware decode: each prompt's 1024-token prefix read once per
    kv-head, with the library's prefix groups."""
    r = run_step(gpu, "prefix_share_fp16", cow_step=cow_step, shared_prefix=True)
    assert len(r["pairs"]) == (224 if cow_step else 0)


@pytest.mark.parametrize("partition", [None, -2])
def test_long_splitk_bf16_full(gpu, partition):
    """The long-context batch with the workload's 512-token partitions and
    with the uniform split (~1100-token partitions, one resident grid)."""
    run_step(gpu, "long_splitk_bf16", partition_tokens=partition)


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
    (where the library writes first); the pool is checked bit for bit and
    every row against the oracle, as for the two-call step."""
    run_step(gpu, name, cow_step=cow_step, partition_tokens=partition, append=True)


def _peak_row(q_row_bits, dtype, head_dim, logit):
    """Bits of a key that is a multiple of the query row, scaled so that its
    logit (q·k/√d) is about ``logit``."""
    qf = to_f64(q_row_bits, dtype)
    alpha = logit * math.sqrt(head_dim) / float(qf @ qf)
    return round_to_bits((qf * alpha).astype(np.float32), dtype)


@pytest.mark.parametrize("partition", [None, -2])
def test_long_splitk_peaked_full_length(gpu, partition):
    """The full-length long-context batch (8 sequences of 32k-131k tokens,
    about 257 partitions of 512 tokens for the longest) with N(0,1) values,
    so scores have a standard deviation of about 1, and three keys of logit
    100 (past 88.7, where fp32 exp overflows without the running max): one in
    the first partition of a sequence, one in a late partition of the longest
    sequence, and one as the new token of a third (its last partition).  The
    tiled softmax's max/sum merge across partitions decides these rows.
    Outputs in fp32, every row compared; the workload's 512-token partitions
    and the uniform split."""
    import torch
    pk = gpu
    st = library_step_state(pk, "long_splitk_bf16")
    w, ora, ids, seed = st["w"], st["ora"], st["ids"], st["seed"]
    dt, G, D, bs = w.dtype, w.group, w.head_dim, w.block_size
    pool = pk.Pool(st["sc"].num_blocks, bs, w.kv_heads, D, dt)
    _fill_and_poison(pool, ora, w, seed + 50, 1.0)
    B = len(ids)
    tdt = torch_dtype(dt)
    q = device_fill_(torch.empty((B, w.q_heads, D), dtype=tdt, device="cuda"), seed + 55, 1.0)
    k_new = device_fill_(torch.empty((B, w.kv_heads, D), dtype=tdt, device="cuda"), seed + 53, 1.0)
    v_new = device_fill_(torch.empty_like(k_new), seed + 54, 1.0)
    q_bits = to_bits(q, dt)
    # the longest sequence is first in dispatch order; positions 1 and 2 take the others
    lens_before = [ora.length(s) for s in ids]
    peaks = [(0, lens_before[0] - 700, 0), (1, 5, 3)]          # (position, token, query row of kv-head 0)
    for pos, tok, row in peaks:
        table, _ = ora.block_table(ids[pos])
        kb = to_torch(_peak_row(q_bits[pos, row], dt, D, 100.0), dt)
        pool.k[int(table[tok // bs]), 0, tok % bs, :] = kb
    k_new[2, 0, :] = to_torch(_peak_row(q_bits[2, 7], dt, D, 100.0), dt)
    k_before, v_before = to_bits(pool.k, dt), to_bits(pool.v, dt)

    step = library_step(st)
    lens = step["lens"]
    pk.write_kv(pool, k_new, v_new, torch.from_numpy(step["slots"]).cuda())
    out = pk.decode(pool, q, torch.from_numpy(step["tables"]).cuda(), torch.from_numpy(lens).cuda(),
                    int(lens.max()), out_dtype="f32",
                    partition_tokens=w.partition_tokens if partition is None else partition)
    torch.cuda.synchronize()
    oracle_write_kv(k_before, v_before, to_bits(k_new, dt), to_bits(v_new, dt), step["o_slots"])
    assert np.array_equal(to_bits(pool.k, dt), k_before) and np.array_equal(to_bits(pool.v, dt), v_before)
    o_tables = np.array(ora.padded_tables(ids, st["stride"], pad=-1), dtype=np.int32)
    want = expected_rows(("long_splitk_bf16", "peaked"), q_bits, k_before, v_before, o_tables, lens.copy(), dt)
    got = out_to_f64(out)
    # the peaked rows are dominated by their key's value row (a sanity check of the case itself)
    for pos, tok, row in peaks + [(2, int(lens[2]) - 1, 7)]:
        table, _ = ora.block_table(ids[pos])
        v_row = to_f64(v_before[int(table[tok // bs]), 0, tok % bs], dt)
        assert np.max(np.abs(want[pos, row] - v_row)) < 1e-6 * max(1.0, float(np.abs(v_row).max())) + 1e-9
    err = np.abs(got - want).reshape(B, -1).max(axis=1)
    print(f"[long peaked, split {partition}] max |err| per sequence {np.array2string(err, precision=2)}",
          flush=True)
    assert float(err.max()) <= TOL[dt]
