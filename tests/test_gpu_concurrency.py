"""Decode calls from two host threads at once, each on its own stream with its
own pool and workspace (the library's contract for calls that may run
concurrently).  The library keeps per-device state only in caches that every
thread fills with the same value and in pa_decode_noalloc's static array
(not used here), so each thread's outputs must equal, bit for bit, what the
same calls give one after the other, and the oracle within tolerance.  ctypes
releases the interpreter lock during the call, so the threads overlap inside
the library.
"""
import threading

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_case, to_torch, out_to_f64, TOL

pytestmark = pytest.mark.gpu

# (lengths, kv_heads, group, block_size, dtype, seed, partition_tokens)
CASES = [
    ([3000, 17, 2500, 1, 900, 0, 1300, 64], 2, 4, 16, "bf16", 41, -2),   # uniform split, matrix-core loop
    ([700, 2047, 33, 1500, 5, 999], 4, 1, 16, "f16", 42, 256),            # fixed partitions, vector loop
]
CALLS = 6


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    return pk


def _setup(pk, lens, kvh, group, bs, dtype, seed, partition):
    import torch
    case = build_case(lens, kvh, group, 128, bs, dtype, seed, scale=1.0)
    pool = pk.Pool(case["num_blocks"], bs, kvh, 128, dtype, k=to_torch(case["k_pool"], dtype),
                   v=to_torch(case["v_pool"], dtype))
    q = to_torch(case["q"], dtype)
    tables = torch.from_numpy(case["tables"]).cuda()
    clens = torch.from_numpy(case["lens"]).cuda()
    max_len = max(lens)
    ws_bytes = pk.decode_workspace_bytes(pool, len(lens), kvh * group, max_len, partition)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    want = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], dtype)
    return dict(pool=pool, q=q, tables=tables, lens=clens, max_len=max_len, ws=ws, partition=partition,
                want=want, dtype=dtype)


def _calls(pk, st, stream, outs):
    import torch
    with torch.cuda.stream(stream):
        for _ in range(CALLS):
            outs.append(pk.decode(st["pool"], st["q"], st["tables"], st["lens"], st["max_len"], out_dtype="f32",
                                  partition_tokens=st["partition"], workspace=st["ws"], stream=stream))


def test_two_threads_decode_at_once(gpu, monkeypatch):
    import torch
    pk = gpu
    monkeypatch.setenv("PA_DEBUG_VALIDATE", "0")   # host validation would synchronise each call
    states = [_setup(pk, *c) for c in CASES]
    streams = [torch.cuda.Stream() for _ in states]
    # one after the other first: the reference bits
    seq = []
    for st, s in zip(states, streams):
        outs = []
        _calls(pk, st, s, outs)
        s.synchronize()
        seq.append(outs[-1].clone())
    # then both threads at once
    results = [[] for _ in states]
    errors = []
    start = threading.Barrier(len(states))

    def run(i):
        try:
            start.wait()
            _calls(pk, states[i], streams[i], results[i])
            streams[i].synchronize()
        except Exception as e:   # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(states))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a decode thread did not finish"
    assert not errors, errors
    for i, st in enumerate(states):
        assert len(results[i]) == CALLS
        for k, got in enumerate(results[i]):
            assert torch.equal(got, seq[i]), f"case {i} call {k}: differs from the sequential run"
        err = np.max(np.abs(out_to_f64(results[i][-1]) - st["want"]))
        print(f"[concurrency] case {i}: {CALLS} calls identical to the sequential run, max |err| {err:.2e}",
              flush=True)
        assert err <= TOL[st["dtype"]]
