"""GPU parity of the benchmark's timed path itself.

bench.py times decode steps that the parity tests elsewhere do not take in
the same way: the batch is re-arranged by the dispatch order every step, the
block manager writes the step's metadata straight into a ring of two pinned
host buffers laid out as one int32 array, one asynchronous copy on a second
stream uploads it into one of two device arrays while the previous step's
kernels run, and the decode calls read their tables, lengths, slots and
groups through views of that array, with host validation off (no host copies or
synchronisation inside the calls).  These tests run that code (the bench's
own build_state, prepare_run and run_steps) for a few steps and check, after
every step, against the oracle's block manager run in lockstep:

* the order the batch was arranged in, and the pinned metadata: slots,
  copy-on-write pairs, padded tables, lengths, prefix groups;
* that the device copy of the metadata (one of two arrays, uploaded on a
  copy stream that overlaps the previous step) equals the pinned bytes;
* the K and V pools of every layer, bit for bit (blocks the step sequence
  touches against the oracle's writes and copies; every other block
  unchanged);
* every output row of the checked layers against the fp64 oracle.

The prompt-scale KV write of the bench's prefill probe is checked bit for bit
as well.
"""
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from oracle.block_manager import OracleBlockManager, NoBlocksError
from oracle.kv_ops import write_kv as oracle_write_kv, copy_blocks as oracle_copy_blocks
from workloads import WORKLOADS, make_scenario
from tests.gpu_util import to_bits, out_to_f64, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    old = os.environ.get("PA_DEBUG_VALIDATE")
    os.environ["PA_DEBUG_VALIDATE"] = "0"      # as the bench runs
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk
    if old is None:
        os.environ.pop("PA_DEBUG_VALIDATE", None)
    else:
        os.environ["PA_DEBUG_VALIDATE"] = old


def _apply(mgr, ops):
    for op in ops:
        if op[0] == "add":
            mgr.add_seq(op[1], op[2])
        elif op[0] == "fork":
            mgr.fork(op[1], op[2])
        else:
            mgr.step(op[1])


def _bits_view(t):
    import torch
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def _poison_dead_slots(pool, ora, bs):
    import torch
    live = np.zeros(pool.num_blocks * bs, dtype=bool)
    for s in ora.seqs:
        live[np.asarray(ora.token_slots(s), dtype=np.int64)] = True
    dead = torch.from_numpy(~live).cuda().view(pool.num_blocks, 1, bs, 1)
    pool.k.masked_fill_(dead, float("nan"))
    pool.v.masked_fill_(dead, float("nan"))


CASES = [
    # workload, batch (None = the workload's), decode entry point, fused append
    ("mha7b_fp16", None, "auto", False),
    ("mha7b_fp16", None, "auto", True),
    ("gqa70b_bf16", 64, "auto", False),
    ("gqa70b_bf16", 64, "auto", True),
    ("prefix_share_fp16", 64, "auto", False),     # prefix groups: pa_decode_shared_prefix
    ("long_splitk_bf16", None, "auto", False),    # 512-token partitions + reduce
    ("long_splitk_bf16", None, "auto", True),
]


@pytest.mark.parametrize("name,batch,decode,fused", CASES)
def test_timed_steps_match_the_oracle(gpu, name, batch, decode, fused):
    import torch
    import bench
    pk = gpu
    w = WORKLOADS[name]
    sc = make_scenario(w, batch=batch)
    layers, n_steps = 2, 3
    st = bench.build_state(pk, w, sc, layers, n_steps)
    run = bench.prepare_run(pk, w, st, 0, decode)
    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    _apply(ora, sc.all_ops())
    for pool in st["pools"]:
        _poison_dead_slots(pool, ora, w.block_size)
    before = [(pool.k.clone(), pool.v.clone()) for pool in st["pools"]]
    torch.cuda.synchronize()
    print(f"[bench path {name}] B={st['B']} layers={layers} steps={n_steps} shared_prefix={run['shared_prefix']} "
          f"fused={fused} split={run['resolved_part']}", flush=True)

    ids = list(sc.measured)
    history = []          # per step: oracle slots, pairs, tables, lens, ids, outputs of the checked layers
    for i in range(n_steps):
        timing = None
        if i == n_steps - 1:   # the timed variant: HIP events around every layer's call (span), or one layer's
            timing = {"used": [], "mode": "span", "every": 1,
                      "free": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                               for _ in range(layers)]}
        bench.run_steps(pk, w, st, 1, run["part"], run["dev"], run["hbufs"], i, timing, run["shared_prefix"], fused)
        torch.cuda.synchronize()
        if timing is not None:   # one span over both layers' calls when each is one pa_decode_append
            spanned = fused and not run["shared_prefix"]
            assert [n for _, _, n, _ in timing["used"]] == ([layers] if spanned else [1])
            assert all(a.elapsed_time(b) > 0 for a, b, _, _ in timing["used"])
        # the oracle takes the same step
        order = ora.dispatch_order(ids)
        ids = [ids[k] for k in order]
        assert [int(x) for x in st["ids"]] == ids, f"step {i}: batch order differs from the oracle's"
        o_slots, o_pairs = ora.step(ids)
        hb = run["hbufs"][i % len(run["hbufs"])]
        assert hb.slots.numpy().tolist() == o_slots, f"step {i}: slots"
        assert hb.pairs.numpy()[:len(o_pairs)].tolist() == [list(p) for p in o_pairs], f"step {i}: pairs"
        o_lens = [ora.length(s) for s in ids]
        o_tables = ora.padded_tables(ids, st["stride"], pad=-1)
        assert hb.lens.numpy().tolist() == o_lens, f"step {i}: lengths"
        assert hb.tables.numpy().tolist() == o_tables, f"step {i}: tables"
        if run["shared_prefix"]:
            starts, prefix, _ = ora.prefix_groups(ids)
            assert hb.group_start.numpy()[:len(starts)].tolist() == starts, f"step {i}: group starts"
            assert hb.prefix.numpy().tolist() == prefix, f"step {i}: prefix tokens"
        meta = run["dev"]["meta"][i % len(run["dev"]["meta"])]
        assert torch.equal(meta["flat"].cpu(), hb.flat), f"step {i}: uploaded metadata differs"
        checked = range(layers) if i == n_steps - 1 else [i % layers]
        outs = {layer: out_to_f64(st["out"][layer]) for layer in checked}
        history.append(dict(slots=o_slots, pairs=o_pairs, tables=np.array(o_tables, dtype=np.int32),
                            lens=np.array(o_lens, dtype=np.int32), outs=outs))

    # blocks the steps read or wrote: every block of every step's tables and every copy source
    touched = sorted({b for h in history for row in h["tables"].tolist() for b in row if b >= 0} |
                     {p[0] for h in history for p in h["pairs"]})
    idx = torch.tensor(touched, dtype=torch.int64, device="cuda")
    for layer, pool in enumerate(st["pools"]):
        k0, v0 = before[layer]
        # blocks outside that set are unchanged
        for now, was in ((pool.k, k0), (pool.v, v0)):
            changed = (_bits_view(now) != _bits_view(was)).view(pool.num_blocks, -1).any(dim=1)
            changed[idx] = False
            assert int(changed.sum()) == 0, f"layer {layer}: a block outside the batch's tables changed"
        # the touched blocks replayed through the oracle, step by step
        shape = (pool.num_blocks, w.kv_heads, w.block_size, w.head_dim)
        bits_t = np.uint32 if w.dtype == "f32" else np.uint16
        k_host, v_host = np.zeros(shape, dtype=bits_t), np.zeros(shape, dtype=bits_t)
        k_host[touched] = to_bits(k0.index_select(0, idx), w.dtype)
        v_host[touched] = to_bits(v0.index_select(0, idx), w.dtype)
        kn, vn = to_bits(st["k_new"][layer], w.dtype), to_bits(st["v_new"][layer], w.dtype)
        q_bits = to_bits(st["q"][layer], w.dtype)
        for i, h in enumerate(history):
            oracle_copy_blocks(k_host, v_host, h["pairs"])
            oracle_write_kv(k_host, v_host, kn, vn, h["slots"])
            if layer in h["outs"]:
                want = paged_decode(q_bits, k_host, v_host, h["tables"], h["lens"], w.dtype)
                err = np.abs(h["outs"][layer] - want).reshape(want.shape[0], -1).max(axis=1)
                print(f"[bench path {name}] step {i} layer {layer}: all {want.shape[0]} rows, "
                      f"max |err| {err.max():.3e}", flush=True)
                assert float(err.max()) <= TOL[w.dtype], f"step {i} layer {layer} row {int(np.argmax(err))}"
        assert np.array_equal(to_bits(pool.k.index_select(0, idx), w.dtype), k_host[touched]), f"layer {layer}: K"
        assert np.array_equal(to_bits(pool.v.index_select(0, idx), w.dtype), v_host[touched]), f"layer {layer}: V"


def test_prefill_probe_write_matches_the_oracle(gpu):
    """The bench's prompt-scale KV write: the library's block manager admits
    the seeded prompts into a fresh 12288-block pool until it is full, and one
    pa_write_kv writes every prompt token (64.6 k rows).  The admitted
    prompts and their slots equal the oracle manager's, and the whole pool
    equals the oracle's write bit for bit."""
    import torch
    import bench
    from paged_kv_cache_355_amd._lib import lib, check
    pk = gpu
    w = WORKLOADS["mha7b_fp16"]
    pool = pk.Pool(w.pool_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    k_want, v_want = to_bits(pool.k, w.dtype), to_bits(pool.v, w.dtype)
    pre = bench.prefill_inputs(pk, w, pool)
    prompts, order = bench.prefill_admission(w, pool.num_blocks)
    ora = OracleBlockManager(pool.num_blocks, w.block_size, order)
    o_slots = []
    for sid, n in prompts[:pre["admitted"]]:
        ora.add_seq(sid, n)
        o_slots.extend(ora.token_slots(sid))
    if pre["admitted"] < len(prompts):   # the library stopped where the oracle runs out of blocks too
        with pytest.raises(NoBlocksError):
            ora.add_seq(*prompts[pre["admitted"]])
    assert pre["slots"].tolist() == o_slots
    n = len(o_slots)
    print(f"[prefill] {pre['admitted']} prompts, {n} tokens", flush=True)
    check(lib().pa_write_kv(pool.handle, pre["k_new"].data_ptr(), pre["v_new"].data_ptr(),
                            pre["slots_dev"].data_ptr(), n, torch.cuda.current_stream().cuda_stream), "pa_write_kv")
    torch.cuda.synchronize()
    oracle_write_kv(k_want, v_want, to_bits(pre["k_new"], w.dtype), to_bits(pre["v_new"], w.dtype), o_slots)
    assert np.array_equal(to_bits(pool.k, w.dtype), k_want)
    assert np.array_equal(to_bits(pool.v, w.dtype), v_want)
