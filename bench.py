"""Throughput of the paged decode hot path on one MI355X.

One timed step is one decode step of a batch of sequences through every
attention layer of a model slice:

1. the host block manager appends one token to each sequence
   (``pa_bm_step``: new block or copy-on-write pair, slot mapping, padded
   block tables and lengths, written into pinned host memory);
2. the metadata goes to the device: one async copy, on a copy stream, into
   one of two device arrays, so it overlaps the previous step's kernels;
3. per layer: ``pa_copy_blocks`` (if the step made copy-on-write pairs),
   then one ``pa_decode_append`` call that writes the new token's K/V into
   its slot and attends over every cached token (``--separate-write``:
   ``pa_write_kv`` then ``pa_decode``).  A batch with prefix groups takes
   ``pa_write_kv`` then ``pa_decode_shared_prefix``.

Each layer has its own KV pool (same block tables, as in a model), so
consecutive decodes never re-read KV that the previous one left in the
256 MB Infinity Cache or the L2s.  All inputs are seeded synthetic values of
the workload's shape, resident in HBM before timing starts.

Printed: one JSON line.  ``value`` is KV bytes read by decode per second of
the whole timed region (host step, copies and kernels included);
``roofline`` is the decode call alone, timed with HIP events on its stream.
When each layer is one library call (``pa_decode_append``), one event pair
brackets the layers' back-to-back calls of every fourth timed step and a call
takes the span divided by the layers; otherwise a pair brackets one layer's
call per step, the layer rotating (``--timed-layers``).  Each recorded pair
leaves the GPU idle for about 5 us on either side;
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same
workload on this host.

    python bench.py [--steps K] [--warmup W] [--layers L] [--workload NAME]
"""
import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_355_amd", "csrc", "decode_impl.h")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=4, help="attention layers per step, one KV pool each")
    ap.add_argument("--workload", default="mha7b_fp16")
    ap.add_argument("--batch", type=int, default=None,
                    help="a smaller batch of the workload's sequences (default: the workload's own batch)")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="0 = the workload's setting (the library's automatic choice unless it names fixed "
                         "partitions); -1 = the balanced split; -2 = the uniform split; > 0 = fixed partitions of "
                         "that many tokens")
    ap.add_argument("--decode", choices=["auto", "plain", "shared"], default="auto",
                    help="auto = pa_decode_shared_prefix when the batch has prefix groups, else pa_decode")
    ap.add_argument("--timed-layers", choices=["span", "one", "all"], default="span",
                    help="decode calls bracketed by HIP events: span (default) = one pair around every layer's "
                         "call of every --timed-every-th step, when each layer is one library call (else as "
                         "'one'); one = one layer's call per step, rotating; all = every layer's call")
    ap.add_argument("--timed-every", type=int, default=4,
                    help="with --timed-layers span: the steps bracketed (every n-th)")
    ap.add_argument("--separate-write", action="store_true",
                    help="pa_write_kv then pa_decode per layer, instead of one pa_decode_append call (the KV write "
                         "inside the decode launch; the default wherever the batch has no prefix groups)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-admission (bulk pa_write_kv) probe")
    ap.add_argument("--no-swap", action="store_true", help="skip the block swap (pa_swap_out / pa_swap_in) probe")
    ap.add_argument("--no-cow", action="store_true", help="skip the copy-on-write (pa_copy_blocks) probe")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="the CPU oracle sample repeats whole steps until this many seconds have passed")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the steps, run a plain elementwise copy of this many MiB three times "
                         "(calibrates HBM byte counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# state
# ----------------------------------------------------------------------------
def build_state(pk, w, sc, layers, steps_total):
    """Block manager with the workload's state, L seeded KV pools and the inputs."""
    import numpy as np
    import torch
    from workloads import device_fill_, seed_for

    bm = pk.BlockManager(sc.num_blocks, w.block_size, sc.free_order)
    for op in sc.all_ops():
        if op[0] == "add":
            bm.add_seq(op[1], op[2])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        else:
            bm.step(op[1])
    ids = np.asarray(sc.measured, dtype=np.int64)
    B = ids.shape[0]
    max_before = max(sc.lengths_before[s] for s in sc.measured)
    stride = -(-(max_before + steps_total) // w.block_size)
    seed = seed_for(w)
    tdt = pk.torch_dtype(w.dtype)
    pools, q, k_new, v_new, out = [], [], [], [], []
    for layer in range(layers):
        pool = pk.Pool(sc.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype)
        base = seed + 100 * layer
        device_fill_(pool.k, base + 1, w.value_scale)
        device_fill_(pool.v, base + 2, w.value_scale)
        pools.append(pool)
        k_new.append(device_fill_(torch.empty((B, w.kv_heads, w.head_dim), dtype=tdt, device="cuda"), base + 3,
                                  w.value_scale))
        v_new.append(device_fill_(torch.empty_like(k_new[-1]), base + 4, w.value_scale))
        q.append(device_fill_(torch.empty((B, w.q_heads, w.head_dim), dtype=tdt, device="cuda"), base + 5,
                              w.value_scale))
        out.append(torch.empty((B, w.q_heads, w.head_dim), dtype=tdt, device="cuda"))
    return dict(bm=bm, ids=ids, B=B, stride=stride, pools=pools, q=q, k_new=k_new, v_new=v_new, out=out)


def meta_len(B, stride):
    return B * (4 + stride) + 2 * B + 1


class HostBuffers:
    """Pinned metadata written by the block manager, laid out as one int32 array
    (slots | lens | copy pairs | block tables | group starts | prefix tokens) so
    a step uploads it in one copy; reused once that copy has left."""

    def __init__(self, B, stride):
        import torch
        self.B, self.stride = B, stride
        self.flat = torch.empty(meta_len(B, stride), dtype=torch.int32, pin_memory=True)
        self.slots, self.lens, self.pairs, self.tables, self.group_start, self.prefix = split_meta(self.flat, B, stride)
        self.lens_np = self.lens.numpy()
        self.prefix_np = self.prefix.numpy()
        self.copied = None   # event recorded after the copy out of these buffers


def split_meta(flat, B, stride):
    """Views (slots[B], lens[B], pairs[B][2], tables[B][stride], group_start[B+1],
    prefix[B]) of one metadata array."""
    t0 = 4 * B
    t1 = t0 + B * stride
    return (flat[:B], flat[B:2 * B], flat[2 * B:4 * B].view(B, 2), flat[t0:t1].view(B, stride),
            flat[t1:t1 + B + 1], flat[t1 + B + 1:t1 + 2 * B + 1])


def prepare_run(pk, w, st, partition_arg=0, decode_arg="auto"):
    """What the timed steps need besides the state: the split (the workload's
    own unless partition_arg is not 0), whether the sharing-aware decode runs
    (decode_arg "auto": when the batch has prefix groups), two device metadata
    arrays with their views (step i uses array i mod 2, uploaded on a copy
    stream while the previous step's kernels run), a zero-filled decode
    workspace sized for the longest context the steps reach, and the two
    pinned host buffers."""
    import torch

    B = st["B"]
    part = w.partition_tokens if partition_arg == 0 else partition_arg
    max_ctx_bound = st["stride"] * w.block_size
    dev = {"meta": [], "copy_stream": torch.cuda.Stream()}
    for _ in range(2):
        m = {"flat": torch.empty(meta_len(B, st["stride"]), dtype=torch.int32, device="cuda"), "free": None}
        (m["slots"], m["lens"], m["pairs"], m["tables"], m["group_start"],
         m["prefix"]) = split_meta(m["flat"], B, st["stride"])
        dev["meta"].append(m)
    # the sharing-aware decode when the batch has prefix groups (and it was not turned off)
    _, probe_prefix, _ = st["bm"].prefix_groups(st["ids"][st["bm"].dispatch_order(st["ids"])])
    shared_prefix = decode_arg == "shared" or (decode_arg == "auto" and int(probe_prefix.max(initial=0)) > 0)
    if shared_prefix and part < 0:
        part = 0
    if shared_prefix:
        ws_bytes = pk.decode_shared_prefix_workspace_bytes(st["pools"][0], B, w.q_heads, max_ctx_bound,
                                                           max_ctx_bound, part)
        resolved_part = part if part > 0 else (
            -(-max_ctx_bound // w.block_size) * w.block_size
            if pk.decode_partition_tokens(st["pools"][0], B, w.q_heads, max_ctx_bound, 0) > 0 else 512)
    else:
        ws_bytes = pk.decode_workspace_bytes(st["pools"][0], B, w.q_heads, max_ctx_bound, part)
        resolved_part = pk.decode_partition_tokens(st["pools"][0], B, w.q_heads, max_ctx_bound, part)
    dev["workspace"] = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")   # counters start at 0
    hbufs = [HostBuffers(B, st["stride"]) for _ in range(2)]
    return {"part": part, "shared_prefix": shared_prefix, "resolved_part": resolved_part, "dev": dev,
            "hbufs": hbufs}


# ----------------------------------------------------------------------------
# the timed step
# ----------------------------------------------------------------------------
def step_timing(timing, fused, n_cow, i):
    """How step i of a run_steps call is bracketed by HIP events: "span" (one
    pair around every layer's call), "one" (one layer's call, rotating), "all"
    (every layer's call) or None.  Span mode applies when each layer is one
    library call (pa_decode_append, no copy-on-write copies before it) and
    takes every timing["every"]-th step counted from the call's first, so any
    run brackets at least one; otherwise it falls back to "one"."""
    if timing is None:
        return None
    if timing["mode"] == "span" and fused and not n_cow:
        return "span" if i % timing["every"] == 0 else None
    return "all" if timing["mode"] == "all" else "one"


def run_steps(pk, w, st, n_steps, partition_tokens, dev, hbufs, step0, timing, shared_prefix, fused_append,
              max_len_override=None):
    """n_steps decode steps; returns per-step KV bytes read by decode.  With
    shared_prefix the batch's prefix groups go to pa_decode_shared_prefix;
    with fused_append each layer's KV write and decode are one
    pa_decode_append call, else pa_write_kv then pa_decode.  max_len_override
    replaces the batch's longest context as the host-known bound (a valid
    bound: every length stays below it)."""
    import numpy as np
    import torch
    from paged_kv_cache_355_amd._lib import lib, check

    L = lib()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    copy_stream = dev["copy_stream"]
    B, stride = st["B"], st["stride"]
    row_bytes = 2 * w.kv_heads * w.head_dim * pk.api.ELEM_BYTES[w.dtype]   # K + V per token
    kv_bytes = []
    for i in range(n_steps):
        hb = hbufs[(step0 + i) % len(hbufs)]
        meta = dev["meta"][(step0 + i) % len(dev["meta"])]
        if hb.copied is not None:
            hb.copied.synchronize()
        # the scheduler arranges the batch for dispatch (long sequences first,
        # prefix siblings adjacent) before the step's metadata is written
        order = st["bm"].dispatch_order(st["ids"])
        if np.any(order != np.arange(B)):
            st["ids"] = np.ascontiguousarray(st["ids"][order])
        n_cow = st["bm"].step_into(st["ids"].ctypes.data, B, hb.slots.data_ptr(), hb.pairs.data_ptr(),
                                   hb.tables.data_ptr(), stride, hb.lens.data_ptr())
        max_len = int(hb.lens_np.max()) if max_len_override is None else max_len_override
        if shared_prefix:
            n_groups, max_group = st["bm"].prefix_groups_into(st["ids"].ctypes.data, B, hb.group_start.data_ptr(),
                                                              hb.prefix.data_ptr())
            max_prefix = int(hb.prefix_np.max())
        # the upload overlaps the previous step's kernels: it waits only for
        # the step that last read this device array, and the decodes wait for it
        if hb.copied is None:
            hb.copied = torch.cuda.Event()
        with torch.cuda.stream(copy_stream):
            if meta["free"] is not None:
                copy_stream.wait_event(meta["free"])
            meta["flat"].copy_(hb.flat, non_blocking=True)
            hb.copied.record(copy_stream)
        stream.wait_event(hb.copied)
        ws = dev["workspace"]
        ws_bytes = ws.numel()
        fused = fused_append and not shared_prefix
        n_layers = len(st["pools"])
        step_mode = step_timing(timing, fused, n_cow, i)
        for layer, pool in enumerate(st["pools"]):
            if n_cow:
                check(L.pa_copy_blocks(pool.handle, meta["pairs"].data_ptr(), n_cow, sptr), "pa_copy_blocks")
            if not fused:
                check(L.pa_write_kv(pool.handle, st["k_new"][layer].data_ptr(), st["v_new"][layer].data_ptr(),
                                    meta["slots"].data_ptr(), B, sptr), "pa_write_kv")
            timed = step_mode == "all" or (step_mode == "one" and layer == (step0 + i) % n_layers)
            if timed or (step_mode == "span" and layer == 0):
                ev0, ev1 = timing["free"].pop()
                ev0.record(stream)
            if shared_prefix:
                check(L.pa_decode_shared_prefix(
                    pool.handle, st["out"][layer].data_ptr(), pk.api.DTYPE_CODES[w.dtype], st["q"][layer].data_ptr(),
                    B, w.q_heads, meta["tables"].data_ptr(), stride, meta["lens"].data_ptr(), max_len, 0.0, n_groups,
                    meta["group_start"].data_ptr(), meta["prefix"].data_ptr(), max_group, max_prefix, partition_tokens,
                    ws.data_ptr(), ws_bytes, sptr), "pa_decode_shared_prefix")
            elif fused:   # the new token's KV write runs inside the decode launch
                check(L.pa_decode_append(pool.handle, st["k_new"][layer].data_ptr(), st["v_new"][layer].data_ptr(),
                                         meta["slots"].data_ptr(), st["out"][layer].data_ptr(),
                                         pk.api.DTYPE_CODES[w.dtype], st["q"][layer].data_ptr(), B, w.q_heads,
                                         meta["tables"].data_ptr(), stride, meta["lens"].data_ptr(), max_len, 0.0,
                                         partition_tokens, ws.data_ptr(), ws_bytes, sptr), "pa_decode_append")
            else:
                check(L.pa_decode(pool.handle, st["out"][layer].data_ptr(), pk.api.DTYPE_CODES[w.dtype],
                                  st["q"][layer].data_ptr(), B, w.q_heads, meta["tables"].data_ptr(), stride,
                                  meta["lens"].data_ptr(), max_len, 0.0, partition_tokens, ws.data_ptr(), ws_bytes,
                                  sptr), "pa_decode")
            if timed:
                ev1.record(stream)
                timing["used"].append((ev0, ev1, 1, i))
            elif step_mode == "span" and layer == n_layers - 1:
                ev1.record(stream)
                timing["used"].append((ev0, ev1, n_layers, i))
        if meta["free"] is None:
            meta["free"] = torch.cuda.Event()
        meta["free"].record(stream)   # this step's kernels are the last readers of meta
        # logical bytes (every sequence's tokens) and unique bytes (each filled slot once:
        # blocks shared by refcount are counted once)
        unique_slots = st["bm"].stats()["filled_slots"]
        kv_bytes.append((int(hb.lens_np.astype("int64").sum()) * row_bytes * len(st["pools"]),
                         int(unique_slots) * row_bytes * len(st["pools"])))
    return kv_bytes


# ----------------------------------------------------------------------------
# memory accounting at the end of the run (the pages' utilisation measures)
# ----------------------------------------------------------------------------
CONTIGUOUS_MAX_LEN = {"mha7b_fp16": 2048, "gqa70b_bf16": 4096, "prefix_share_fp16": 2048,
                      "long_splitk_bf16": 131072, "tiny_fp32": 16}


def memory_accounting(bm, w):
    """Slots holding a token ÷ slots reserved, for the paged pool (from the block
    manager's counters) and for a contiguous reservation of the workload's maximum
    length per sequence; and logical ÷ physical blocks (sharing)."""
    st = bm.stats()
    max_len = CONTIGUOUS_MAX_LEN.get(w.name, 0)
    paged = st["filled_slots"] / max(1, st["used_blocks"] * st["block_size"])
    contiguous = st["logical_tokens"] / max(1, st["num_seqs"] * max_len) if max_len else None
    return {"paged_slot_utilisation": round(paged, 4),
            "contiguous_slot_utilisation": None if contiguous is None else round(contiguous, 4),
            "contiguous_max_len": max_len,
            "logical_over_physical_blocks": round(st["logical_blocks"] / max(1, st["used_blocks"]), 3),
            "used_blocks": st["used_blocks"], "pool_blocks": st["num_blocks"]}


# ----------------------------------------------------------------------------
# CPU oracle sample
# ----------------------------------------------------------------------------
def cpu_baseline(w, sc, budget_s):
    """The oracle's full step (block manager, KV write, fp64 decode) for one layer of
    the same batch, repeated while the time budget lasts (at least once)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle.attention import paged_decode
    from oracle.block_manager import OracleBlockManager
    from oracle.kv_ops import write_kv as oracle_write_kv, copy_blocks as oracle_copy_blocks
    from oracle.numerics import bits_dtype, elem_bytes

    ora = OracleBlockManager(sc.num_blocks, w.block_size, sc.free_order)
    for op in sc.all_ops():
        if op[0] == "add":
            ora.add_seq(op[1], op[2])
        elif op[0] == "fork":
            ora.fork(op[1], op[2])
        else:
            ora.step(op[1])
    ids = list(sc.measured)
    rng = np.random.default_rng(12345)
    bt = bits_dtype(w.dtype)
    shape = (sc.num_blocks, w.kv_heads, w.block_size, w.head_dim)
    # finite small values in every block (bit patterns of |x| < 1); values do not change the oracle's cost
    limit = 0x3F800000 if w.dtype == "f32" else (0x3C00 if w.dtype == "f16" else 0x3F80)
    k_pool = np.zeros(shape, dtype=bt)
    v_pool = np.zeros(shape, dtype=bt)
    used = np.array(sorted({b for s in ids for b in ora.block_table(s)[0]}), dtype=np.int64)
    tile = rng.integers(0, limit, size=(256,) + shape[1:], dtype=bt)
    k_pool[used] = tile[np.arange(used.shape[0]) % 256]
    v_pool[used] = tile[(np.arange(used.shape[0]) + 128) % 256]
    q = rng.integers(0, limit, size=(len(ids), w.q_heads, w.head_dim), dtype=bt)
    k_new = rng.integers(0, limit, size=(len(ids), w.kv_heads, w.head_dim), dtype=bt)
    v_new = rng.integers(0, limit, size=(len(ids), w.kv_heads, w.head_dim), dtype=bt)
    row_bytes = 2 * w.kv_heads * w.head_dim * elem_bytes(w.dtype)
    times, kv = [], []
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        while not times or time.perf_counter() - t_start < budget_s:
            t0 = time.perf_counter()
            slots, pairs = ora.step(ids)
            oracle_copy_blocks(k_pool, v_pool, pairs)
            oracle_write_kv(k_pool, v_pool, k_new, v_new, slots)
            lens = np.array([ora.length(s) for s in ids], dtype=np.int64)
            stride = -(-int(lens.max()) // w.block_size)
            tables = np.array(ora.padded_tables(ids, stride, pad=0), dtype=np.int32)
            paged_decode(q, k_pool, v_pool, tables, lens, w.dtype)
            times.append(time.perf_counter() - t0)
            kv.append(int(lens.sum()) * row_bytes)
    t = sum(times)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(sum(kv) / t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(times)} full decode step(s) of the {len(ids)}-sequence batch through one layer "
                  f"(block manager step, KV write, fp64 paged decode), single-threaded numpy",
        "seq_steps_per_s": round(len(ids) * len(times) / t, 3),
        "seconds": round(t, 3),
        "host_cpu": cpu_model,
        "host_cpus_available": os.cpu_count(),
    }


# ----------------------------------------------------------------------------
# HBM traffic recorded from rocprofv3 counters for this kernel source
# ----------------------------------------------------------------------------
def kernel_source_hash():
    """sha256[:16] of the decode kernels' code with // comments and blank
    space removed, so an edit of comments alone keeps recorded counters valid."""
    code = []
    with open(KERNEL_SOURCE, encoding="utf-8") as f:
        for line in f:
            line = re.sub(r"//.*$", "", line).strip()
            if line:
                code.append(re.sub(r"\s+", " ", line))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def recorded_traffic(workload, decode):
    """(HBM bytes per decode call, their ratio to the algorithmic bytes of the
    counted run) from the committed counter summary, if it was taken on the
    current kernel source with the same decode entry point (else (None, None))."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None, None
    rec = None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            rec = json.loads(line)
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("decode", "pa_decode") != decode:
        return None, None
    return rec.get("hbm_bytes_per_call"), round(rec["hbm_bytes_per_call"] / rec["algorithmic_bytes_per_call"], 4)


def prefill_admission(w, num_blocks):
    """The prompts the prefill probe admits (a second seeded draw of the
    workload's prompts, (seq id, tokens) in admission order) and the free-list
    order of its fresh block manager."""
    import numpy as np
    from workloads import make_scenario, seed_for

    sc2 = make_scenario(w, repetition=1)
    prompts = [(op[1], op[2]) for op in sc2.setup if op[0] == "add"]
    return prompts, np.random.default_rng(seed_for(w, 1)).permutation(num_blocks)


def prefill_inputs(pk, w, pool):
    """A fresh block manager over ``pool`` admits the prefill prompts until the
    pool is full (add_seq, then each prompt's token slots); returns the slots
    of every admitted prompt token and seeded K/V rows for them on the device."""
    import numpy as np
    import torch
    from workloads import device_fill_, seed_for

    prompts, order = prefill_admission(w, pool.num_blocks)
    t0 = time.perf_counter()
    bm = pk.BlockManager(pool.num_blocks, w.block_size, order)
    slots = []
    admitted = 0
    for sid, n in prompts:
        try:
            bm.add_seq(sid, n)
        except pk.NoBlocksError:
            break
        slots.append(bm.token_slots(sid, 0, n))
        admitted += 1
    slots = np.concatenate(slots).astype(np.int32)
    host_ms = (time.perf_counter() - t0) * 1e3
    n_tok = int(slots.shape[0])
    seed = seed_for(w, 1)
    tdt = pk.torch_dtype(w.dtype)
    k_new = device_fill_(torch.empty((n_tok, w.kv_heads, w.head_dim), dtype=tdt, device="cuda"), seed + 11,
                         w.value_scale)
    v_new = device_fill_(torch.empty_like(k_new), seed + 12, w.value_scale)
    return {"bm": bm, "admitted": admitted, "slots": slots, "slots_dev": torch.from_numpy(slots).cuda(),
            "k_new": k_new, "v_new": v_new, "host_admit_ms": host_ms}


def prefill_probe(pk, w, st, reps=5):
    """Prompt admission at prompt scale: a fresh block manager over the first
    layer's pool admits a second seeded draw of the workload's prompts
    (add_seq, then each prompt's token slots), and one bulk pa_write_kv writes
    every prompt token's K and V (partial last blocks included).  Runs after
    the timed decode steps, whose pool contents it overwrites."""
    import torch
    from paged_kv_cache_355_amd._lib import lib, check

    pool = st["pools"][0]
    pre = prefill_inputs(pk, w, pool)
    host_ms = pre["host_admit_ms"]
    admitted, k_new, v_new, slots_dev = pre["admitted"], pre["k_new"], pre["v_new"], pre["slots_dev"]
    n_tok = int(pre["slots"].shape[0])
    stream = torch.cuda.current_stream()
    L = lib()
    args = (pool.handle, k_new.data_ptr(), v_new.data_ptr(), slots_dev.data_ptr(), n_tok, stream.cuda_stream)
    check(L.pa_write_kv(*args), "pa_write_kv")   # warm-up (re-writing the same slots is idempotent)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        check(L.pa_write_kv(*args), "pa_write_kv")
        e1.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    moved = 2 * 2 * n_tok * w.kv_heads * w.head_dim * pk.api.ELEM_BYTES[w.dtype]   # K and V, read + write
    del k_new, v_new, slots_dev
    return {"prompts": admitted, "tokens": n_tok, "host_admit_ms": round(host_ms, 3),
            "write_kv_us": round(us, 2), "write_kv_GBps": round(moved / us / 1e3, 1),
            "frac_of_hbm_peak": round(moved / us / 1e3 / HBM_PEAK_GBPS, 4),
            "bytes": "K and V of every prompt token, read from the staging tensors and written into the pool"}


def cow_probe(pk, w, st, reps=5):
    """Copy-on-write at a fork: the prefix-sharing workload's first step after
    the fork copies every shared, part-filled last block (pa_bm_step's pairs,
    224 for 32 prompts x 8 samples).  A workload without forks copies each
    sequence's last block into a free block, as a fork of the whole batch
    would.  pa_copy_blocks on the first layer's pool; repeating the same
    pairs is idempotent."""
    import numpy as np
    import torch
    from paged_kv_cache_355_amd._lib import lib, check
    from workloads import make_scenario

    pool = st["pools"][0]
    sc = make_scenario(w)
    if sc.cow_step is not None:
        bm = pk.BlockManager(sc.num_blocks, w.block_size, sc.free_order)
        for op in sc.setup:
            if op[0] == "add":
                bm.add_seq(op[1], op[2])
            else:
                bm.fork(op[1], op[2])
        pairs = bm.step(sc.cow_step)[1]
        source = "the fork step's copy-on-write pairs (pa_bm_step)"
    else:
        free = st["bm"].free_list()
        last = [st["bm"].block_table(s)[0][-1] for s in st["ids"][:len(free)]]
        pairs = np.stack([np.asarray(last, dtype=np.int32), np.asarray(free[:len(last)], dtype=np.int32)], axis=1)
        source = "each sequence's last block into a free block"
    n = int(pairs.shape[0])
    if n == 0:
        return None
    pairs_dev = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).cuda()
    stream = torch.cuda.current_stream()
    L = lib()
    check(L.pa_copy_blocks(pool.handle, pairs_dev.data_ptr(), n, stream.cuda_stream), "pa_copy_blocks")   # warm-up
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        check(L.pa_copy_blocks(pool.handle, pairs_dev.data_ptr(), n, stream.cuda_stream), "pa_copy_blocks")
        e1.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    moved = 2 * 2 * n * pool.block_bytes   # K and V blocks, read + written
    sources = int(np.unique(pairs[:, 0]).shape[0])
    unique = 2 * (sources + n) * pool.block_bytes   # each source read once, each destination written
    return {"pairs": n, "distinct_sources": sources, "pairs_from": source, "copy_blocks_us": round(us, 2),
            "copy_blocks_GBps": round(moved / us / 1e3, 1), "unique_GBps": round(unique / us / 1e3, 1),
            "unique_frac_of_hbm_peak": round(unique / us / 1e3 / HBM_PEAK_GBPS, 4),
            "bytes": "copy_blocks_GBps: K and V of every pair's source read and destination written; "
                     "unique_GBps: each distinct source read once (a shared block's later copies hit cache)"}


def stream_read_probe(gib=2, reps=10):
    """A plain streaming read measured on this GPU: torch's sum over a 2 GiB
    buffer viewed as int64 (default cache policy), the median of reps calls."""
    import torch
    n = gib << 30
    x = torch.ones(n // 8, dtype=torch.int64, device="cuda")
    for _ in range(3):
        x.sum()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        x.sum()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    del x
    return round(n / (ms * 1e-3) / 1e9, 1)


def swap_probe(pk, st, target_mib=256, reps=3):
    """Block swap between the first layer's pool and pinned host memory: about
    target_mib MiB of whole blocks out (pa_swap_out) and back into the same
    blocks (pa_swap_in, which restores the bytes it just saved)."""
    import torch
    from paged_kv_cache_355_amd._lib import lib, check

    pool = st["pools"][0]
    per_block = 2 * pool.block_bytes
    n = max(1, min(pool.num_blocks, (target_mib << 20) // per_block))
    blocks = torch.arange(n, dtype=torch.int32, device="cuda")
    host = torch.empty(n * per_block, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()
    L = lib()
    res = {}
    for name, fn in (("out", L.pa_swap_out), ("in", L.pa_swap_in)):
        args = (pool.handle, blocks.data_ptr(), n, host.data_ptr(), n * per_block, stream.cuda_stream)
        check(fn(*args), f"pa_swap_{name}")   # warm-up
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            check(fn(*args), f"pa_swap_{name}")
            e1.record(stream)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
        res[f"swap_{name}_us"] = round(us, 1)
        res[f"swap_{name}_GBps"] = round(n * per_block / us / 1e3, 2)
    res.update({"blocks": n, "bytes": n * per_block,
                "path": "one kernel between HBM and pinned host memory, no staging copy"})
    return res


def copy_probe(mib):
    """A plain elementwise kernel of known traffic (reads and writes mib MiB)."""
    import torch
    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log(f"copy probe: 3 x torch.neg over {mib} MiB fp16 (reads {mib} MiB, writes {mib} MiB per dispatch)")


# ----------------------------------------------------------------------------
def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode path shards by sequence or kv-head with no exchange; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import paged_kv_cache_355_amd as pk
    from workloads import WORKLOADS, make_scenario

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pk.lib()
    w = WORKLOADS[args.workload]
    sc = make_scenario(w, batch=args.batch)
    steps_total = args.warmup + args.steps
    log(f"[bench] workload {w.name}: B={len(sc.measured)} Hq={w.q_heads} Hkv={w.kv_heads} d={w.head_dim} "
        f"{w.dtype} bs={w.block_size} pool={sc.num_blocks} blocks x {args.layers} layers")
    st = build_state(pk, w, sc, args.layers, steps_total)
    B = st["B"]
    run = prepare_run(pk, w, st, args.partition_tokens, args.decode)
    part, shared_prefix, resolved_part = run["part"], run["shared_prefix"], run["resolved_part"]
    dev, hbufs = run["dev"], run["hbufs"]
    max_ctx_bound = st["stride"] * w.block_size
    torch.cuda.synchronize()
    log(f"[bench] state ready; warmup {args.warmup} steps")

    fused_append = not args.separate_write
    # The last warmup step takes the longest context the steps can reach as
    # its bound: it launches every kernel variant the timed steps may need (a
    # split and its reduce start once contexts grow past a partition), so none
    # is loaded for the first time inside the timed region.
    if args.warmup > 1:
        run_steps(pk, w, st, args.warmup - 1, part, dev, hbufs, 0, None, shared_prefix, fused_append)
    if args.warmup > 0:
        run_steps(pk, w, st, 1, part, dev, hbufs, args.warmup - 1, None, shared_prefix, fused_append,
                  max_len_override=max_ctx_bound)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    # HIP events on the launch stream: each recorded pair leaves the GPU idle
    # for about 5 us on either side, so by default one pair brackets the
    # layers' back-to-back calls of every fourth step (--timed-layers)
    timing = {"used": [], "mode": args.timed_layers, "every": max(1, args.timed_every),
              "free": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.steps * args.layers)]}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kv_bytes = run_steps(pk, w, st, args.steps, part, dev, hbufs, args.warmup, timing, shared_prefix,
                         fused_append)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    spans = [(a.elapsed_time(b), n, i) for a, b, n, i in timing["used"]]   # (ms, calls bracketed, step)
    dec_ms = [ms / n for ms, n, _ in spans]   # one call's duration per sample
    log(f"[bench] done: {elapsed * 1e3:.2f} ms for {args.steps} steps")

    total_kv = sum(b for b, _ in kv_bytes)
    total_unique = sum(u for _, u in kv_bytes)
    layers = len(st["pools"])
    # every layer's decode reads the same tokens (same tables and lengths);
    # the minimum traffic counts shared blocks once
    per_call_bytes = total_unique / (args.steps * layers)
    # the bracketed calls' own bytes (lengths grow by one token per step) over their time
    achieved = (sum(kv_bytes[i][1] / layers * n for _, n, i in spans) /
                (sum(ms for ms, _, _ in spans) / 1e3) / 1e9)
    mean_dec_s = sum(ms for ms, _, _ in spans) / sum(n for _, n, _ in spans) / 1e3
    timing_note = (f"one HIP event pair around the {layers} layers' back-to-back decode calls of every "
                   f"{timing['every']}th step ({len(spans)} spans), per call = span / {layers}"
                   if all(n == layers for _, n, _ in spans) and layers > 1 else
                   "one HIP event pair around each layer's decode call" if args.timed_layers == "all" else
                   "one HIP event pair around one layer's decode call per step, the layer rotating")
    value = total_kv / elapsed / 1e9
    entry = "pa_decode_shared_prefix" if shared_prefix else ("pa_decode_append" if fused_append else "pa_decode")
    traffic, traffic_ratio = recorded_traffic(w.name, entry)
    dec_sorted = sorted(dec_ms)
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + seq-steps/s, 7B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "pool_blocks": sc.num_blocks,
            "layers_per_step": layers, "partition_tokens": resolved_part,
            "decode": entry,
            "context_lens": "uniform [128, 2048] before the first warmup step, +1 per step"
            if w.name == "mha7b_fp16" else w.notes,
            "mean_context_len_timed": round(total_kv / (args.steps * layers * 2 * w.kv_heads * w.head_dim *
                                                        pk.api.ELEM_BYTES[w.dtype]) / B, 1),
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "unique_kv_GBps": round(total_unique / elapsed / 1e9, 2),
        "seq_steps_per_s_per_layer": round(B * layers * args.steps / elapsed, 1),
        "decode_call_us": {"mean": round(mean_dec_s * 1e6, 2),
                           "p10": round(dec_sorted[len(dec_sorted) // 10] * 1e3, 2),
                           "p50": round(dec_sorted[len(dec_sorted) // 2] * 1e3, 2),
                           "p90": round(dec_sorted[(9 * len(dec_sorted)) // 10] * 1e3, 2),
                           "events": timing_note},
        "roofline": {
            "kernel": ("pa_decode_shared_prefix: decode_prefix_kernel + decode_partition_kernel" +
                       (" + decode_reduce_kernel" if resolved_part < max_ctx_bound else "") if shared_prefix else
                       entry + (": write_kv_kernel + decode_balanced_kernel" if entry == "pa_decode_append"
                                else ": decode_balanced_kernel") if resolved_part == -1 else
                       entry + ": decode_uniform_kernel + decode_reduce_kernel (uniform split)"
                       if resolved_part == -2 else
                       entry + ": decode_partition_kernel" + (" + decode_reduce_kernel"
                                                               if resolved_part < max_ctx_bound else
                                                               " (one workgroup per sequence and kv-head)")),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            # HBM bytes per call of this run: the ratio that the committed
            # FETCH_SIZE/WRITE_SIZE runs measured for this kernel source and
            # entry point, times this run's algorithmic bytes per call
            "traffic": None if traffic_ratio is None else int(round(traffic_ratio * per_call_bytes)),
            "traffic_over_algorithmic": traffic_ratio,
            "traffic_source": None if traffic_ratio is None else
            f"profiles/decode_{w.name}_traffic.txt (counted {traffic} B per call on shorter contexts)",
            "algorithmic_bytes_per_call": int(per_call_bytes),
        },
        "cpu_baseline": None,
    }
    result["memory"] = memory_accounting(st["bm"], w)
    if not args.no_prefill:
        result["prefill"] = prefill_probe(pk, w, st)
    if not args.no_swap:
        result["swap"] = swap_probe(pk, st)
    if not args.no_cow:
        result["copy_on_write"] = cow_probe(pk, w, st)
    if not args.no_read_probe:
        read_gbps = stream_read_probe()
        result["stream_read_probe"] = {"GBps": read_gbps, "decode_over_probe": round(achieved / read_gbps, 4),
                                       "kernel": "torch.sum over a 2 GiB buffer viewed as int64 (default cache "
                                                 "policy), median of 10; a measured streaming-read rate of this GPU"}
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle sample (budget {args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, sc, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
