"""pa_decode_noalloc: pa_decode without a workspace, for callers that cannot
allocate device memory.  Called through the C ABI, it must give what
pa_decode gives with a caller workspace (the same kernels on the same split:
bit for bit), and the fp64 oracle's result, on consecutive calls of
different sizes that share the library's static array; splits that do not
fit the array are refused before anything runs."""
import ctypes
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_case, to_torch, out_to_f64, TOL

pytestmark = pytest.mark.gpu

STATIC_BYTES = 16 << 20


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def _noalloc(pk, pool, out, q, tables, lens, max_len, partition):
    """pa_decode_noalloc through the C ABI; returns its status."""
    import torch
    from paged_kv_cache_355_amd._lib import lib
    B, hq, _ = q.shape
    return lib().pa_decode_noalloc(pool.handle, out.data_ptr(), pk.api.DTYPE_CODES["f32"], q.data_ptr(), B, hq,
                                   tables.data_ptr(), int(tables.shape[1]), lens.data_ptr(), max_len,
                                   ctypes.c_float(0.0), partition, torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_pa_decode_on_consecutive_calls(gpu):
    """Three calls in a row on one GPU, each smaller than the one before:
    fixed 256-token partitions over 12 sequences (partial records in the
    static array), the balanced split over 7 (its merge counters there too,
    cleared by the call), the uniform split over 3.  Each equals pa_decode
    with a zero-filled caller workspace bit for bit and the oracle within
    2e-3; a whole-sequence call (no partial results) as well."""
    import torch
    from paged_kv_cache_355_amd._lib import check
    pk = gpu
    lens = [3000, 17, 2500, 1, 900, 0, 1300, 64, 2047, 700, 16, 1999]
    case = build_case(lens, 2, 4, 128, 16, "f16", 91, scale=1.0)
    want = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], "f16")
    pool = pk.Pool(case["num_blocks"], 16, 2, 128, "f16", k=to_torch(case["k_pool"], "f16"),
                   v=to_torch(case["v_pool"], "f16"))
    q_all = to_torch(case["q"], "f16")
    tables_all = torch.from_numpy(case["tables"]).cuda()
    lens_all = torch.from_numpy(case["lens"]).cuda()
    bal, uni = pk.PA_PARTITION_BALANCED, pk.PA_PARTITION_UNIFORM
    calls = [(12, 256), (7, bal), (3, uni), (12, 4096)]
    for n, partition in calls:
        q, tables, lens_n = q_all[:n].contiguous(), tables_all[:n].contiguous(), lens_all[:n].contiguous()
        max_len = int(case["lens"][:n].max())
        need = pk.decode_workspace_bytes(pool, n, 8, max_len, partition)
        assert need <= STATIC_BYTES
        out = torch.full((n, 8, 128), float("nan"), dtype=torch.float32, device="cuda")
        check(_noalloc(pk, pool, out, q, tables, lens_n, max_len, partition), "pa_decode_noalloc")
        torch.cuda.synchronize()
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        ref = pk.decode(pool, q, tables, lens_n, max_len, out_dtype="f32", partition_tokens=partition, workspace=ws)
        torch.cuda.synchronize()
        print(f"[noalloc] {n} seqs, split {partition}, {need} workspace bytes", flush=True)
        assert torch.equal(out, ref), f"split {partition}: differs from pa_decode"
        assert np.max(np.abs(out_to_f64(out) - want[:n])) <= TOL["f16"], f"split {partition}: differs from the oracle"


def test_noalloc_refuses_a_split_beyond_its_array(gpu):
    """64 sequences x 32 heads in 16-token partitions of a 2048-token context
    keep ~136 MB of partial results: refused with PA_ERR_INVALID and a message,
    nothing launched (the output keeps its contents)."""
    import torch
    from paged_kv_cache_355_amd._lib import lib, PA_ERR_INVALID
    pk = gpu
    pool = pk.Pool(64 * 128 + 1, 16, 32, 128, "f16")
    B = 64
    assert pk.decode_workspace_bytes(pool, B, 32, 2048, 16) > STATIC_BYTES
    q = torch.zeros((B, 32, 128), dtype=torch.float16, device="cuda")
    tables = torch.arange(B * 128, dtype=torch.int32, device="cuda").view(B, 128)
    lens = torch.full((B,), 2048, dtype=torch.int32, device="cuda")
    out = torch.full((B, 32, 128), 7.0, dtype=torch.float32, device="cuda")
    code = _noalloc(pk, pool, out, q, tables, lens, 2048, 16)
    torch.cuda.synchronize()
    assert code == PA_ERR_INVALID
    assert "pa_decode_noalloc holds" in lib().pa_last_error().decode()
    assert bool((out == 7.0).all())
