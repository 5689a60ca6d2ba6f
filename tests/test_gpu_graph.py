"""Decode calls captured into a HIP graph (torch.cuda.graph) and replayed.

pa_decode_noalloc exists for callers that cannot allocate, code under graph
capture among them: it takes no workspace, and the balanced split's counters
in the library's static array are cleared by a fill kernel (no memset node).
Each case captures one call, then replays the graph four times; before each
replay the query changes (eager work on the stream), and every replay must
give, bit for bit, what the same call gives eagerly on the same inputs.  The
fused KV write (pa_decode_append) is captured too: its replays rewrite the
same slot with the same row.
"""
import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_case, to_torch, to_bits, out_to_f64, TOL

pytestmark = pytest.mark.gpu

LENS = [3000, 17, 2500, 1, 900, 0, 1300, 64, 2047, 700, 16, 1999]


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    return pk


def _case(pk):
    case = build_case(LENS, 2, 4, 128, 16, "f16", 123, scale=1.0)
    pool = pk.Pool(case["num_blocks"], 16, 2, 128, "f16", k=to_torch(case["k_pool"], "f16"),
                   v=to_torch(case["v_pool"], "f16"))
    return case, pool


@pytest.mark.parametrize("partition", [256, -1, -2], ids=["fixed256", "balanced", "uniform"])
def test_noalloc_graph_replays_match_eager(gpu, monkeypatch, partition):
    import torch
    pk = gpu
    monkeypatch.setenv("PA_DEBUG_VALIDATE", "0")   # host validation synchronises, which capture forbids
    case, pool = _case(pk)
    q = to_torch(case["q"], "f16")
    tables = torch.from_numpy(case["tables"]).cuda()
    lens = torch.from_numpy(case["lens"]).cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")

    def call(o):
        pk.decode_noalloc(pool, q, tables, lens, 3000, out=o, out_dtype="f32", partition_tokens=partition)

    call(out)                  # eager first: kernels loaded, the library's per-device lookups made
    torch.cuda.synchronize()
    want = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], "f16")
    assert np.max(np.abs(out_to_f64(out) - want)) <= TOL["f16"]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    ref = torch.empty_like(out)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for k in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.float16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call(ref)              # the same call, eagerly, on the same inputs
        torch.cuda.synchronize()
        print(f"[graph] partition {partition} replay {k}: identical {torch.equal(got, ref)}", flush=True)
        assert torch.equal(got, ref), f"replay {k}"


def test_append_graph_replays_match_eager(gpu, monkeypatch):
    """pa_decode_append (whole sequences, no workspace) under capture: every
    replay writes the new rows into their slots and attends over them."""
    import torch
    pk = gpu
    monkeypatch.setenv("PA_DEBUG_VALIDATE", "0")
    case, pool = _case(pk)
    B = len(LENS)
    q = to_torch(case["q"], "f16")
    tables = torch.from_numpy(case["tables"]).cuda()
    lens_np = case["lens"].copy()
    # the appended token is each non-empty sequence's last: its slot from the table
    slots = np.array([int(case["tables"][s][(n - 1) // 16]) * 16 + (n - 1) % 16 if n > 0 else -1
                      for s, n in enumerate(lens_np)], dtype=np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    slot_t = torch.from_numpy(slots).cuda()
    gen = torch.Generator(device="cuda").manual_seed(11)
    k_new = torch.randn((B, 2, 128), generator=gen, device="cuda").to(torch.float16)
    v_new = torch.randn((B, 2, 128), generator=gen, device="cuda").to(torch.float16)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")

    def call(o):
        pk.decode(pool, q, tables, lens, 3000, out=o, out_dtype="f32", partition_tokens=3008,
                  append=(k_new, v_new, slot_t))

    call(out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    ref = torch.empty_like(out)
    for k in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.float16))
        k_new.copy_(torch.randn(k_new.shape, generator=gen, device="cuda").to(torch.float16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        pool_k = pool.k.clone()
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {k}: outputs"
        # bit patterns: the pool's padding slots hold NaN
        assert torch.equal(pool_k.view(torch.int16), pool.k.view(torch.int16)), f"replay {k}: pool"
        # the replay itself wrote this replay's new rows into their slots
        for s in range(B):
            if slots[s] >= 0:
                blk, off = divmod(int(slots[s]), 16)
                assert torch.equal(pool_k[blk, :, off, :].view(torch.int16), k_new[s].view(torch.int16)), \
                    f"replay {k}: slot of sequence {s}"


def test_whole_decode_step_graph_replays_match_eager(gpu, monkeypatch):
    """One decode step captured whole: the upload of the step's metadata
    (slots, lengths, block tables) from pinned host memory, then
    pa_decode_append for two layers.  Before each replay the library's block
    manager writes the next step's metadata into the same pinned buffer; the
    replay uploads it, writes the new tokens and decodes.  The same calls run
    eagerly on a copy of the pools must give the same outputs and pools, bit
    for bit, and the last step's outputs match the oracle."""
    import torch
    pk = gpu
    monkeypatch.setenv("PA_DEBUG_VALIDATE", "0")
    B, bs, kvh, G, d, dt, layers, steps = 6, 16, 2, 4, 128, "bf16", 2, 4
    nb = 256
    lens0 = [700, 3, 1500, 64, 1, 999]
    bm = pk.BlockManager(nb, bs, np.random.default_rng(31).permutation(nb))
    for s, n in enumerate(lens0):
        bm.add_seq(s, n)
    ids = np.arange(B, dtype=np.int64)
    stride = -(-(max(lens0) + steps + 1) // bs)
    max_ctx = stride * bs                      # every step's lengths stay under it: one partition per unit
    tdt = pk.torch_dtype(dt)
    gen = torch.Generator(device="cuda").manual_seed(5)

    def rand(*shape):
        return (torch.randn(shape, generator=gen, device="cuda") / 11.3).to(tdt)

    pools_g = [pk.Pool(nb, bs, kvh, d, dt) for _ in range(layers)]
    for p in pools_g:
        p.k.copy_(rand(*p.k.shape))
        p.v.copy_(rand(*p.v.shape))
    pools_e = [pk.Pool(nb, bs, kvh, d, dt, k=p.k.clone(), v=p.v.clone()) for p in pools_g]
    q = [rand(B, kvh * G, d) for _ in range(layers)]
    k_new = [rand(B, kvh, d) for _ in range(layers)]
    v_new = [rand(B, kvh, d) for _ in range(layers)]
    n_meta = 2 * B + B * stride                # slots | lengths | tables
    host = torch.empty(n_meta, dtype=torch.int32, pin_memory=True)
    dev_g = torch.empty(n_meta, dtype=torch.int32, device="cuda")
    dev_e = torch.empty_like(dev_g)
    pairs = np.zeros((B, 2), dtype=np.int32)

    def views(t):
        return t[:B], t[B:2 * B], t[2 * B:].view(B, stride)

    def host_step():
        h_slots, h_lens, h_tables = views(host)
        n_cow = bm.step_into(ids.ctypes.data, B, h_slots.data_ptr(), pairs.ctypes.data, h_tables.data_ptr(), stride,
                             h_lens.data_ptr())
        assert n_cow == 0

    def layers_of(pools, outs, meta):
        slots, lens, tables = views(meta)
        for l in range(layers):
            pk.decode(pools[l], q[l], tables, lens, max_ctx, out=outs[l], out_dtype="f32", partition_tokens=max_ctx,
                      append=(k_new[l], v_new[l], slots))

    outs_g = [torch.empty((B, kvh * G, d), dtype=torch.float32, device="cuda") for _ in range(layers)]
    outs_e = [torch.empty_like(o) for o in outs_g]
    host_step()                                # step 1, eager on both copies (kernels loaded)
    dev_g.copy_(host)
    layers_of(pools_g, outs_g, dev_g)
    dev_e.copy_(host)
    layers_of(pools_e, outs_e, dev_e)
    torch.cuda.synchronize()
    host_step()                                # step 2's metadata, uploaded by the graph itself
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev_g.copy_(host, non_blocking=True)
        layers_of(pools_g, outs_g, dev_g)
    for step in range(2, steps + 1):
        if step > 2:
            host_step()
        graph.replay()
        torch.cuda.synchronize()
        dev_e.copy_(host)
        layers_of(pools_e, outs_e, dev_e)
        torch.cuda.synchronize()
        assert torch.equal(dev_g, dev_e), f"step {step}: uploaded metadata"
        for l in range(layers):
            assert torch.equal(outs_g[l], outs_e[l]), f"step {step} layer {l}: outputs"
            for a, b in ((pools_g[l].k, pools_e[l].k), (pools_g[l].v, pools_e[l].v)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"step {step} layer {l}: pool"
        print(f"[graph step] step {step}: replay identical to eager", flush=True)
    _, lens_t, tables_t = views(dev_e)
    for l in range(layers):
        want = paged_decode(to_bits(q[l], dt), to_bits(pools_e[l].k, dt), to_bits(pools_e[l].v, dt),
                            tables_t.cpu().numpy(), lens_t.cpu().numpy(), dt)
        assert np.max(np.abs(out_to_f64(outs_g[l]) - want)) <= TOL[dt]
