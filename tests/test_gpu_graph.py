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
from tests.gpu_util import build_case, to_torch, out_to_f64, TOL

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
