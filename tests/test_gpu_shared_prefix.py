"""GPU parity of the sharing-aware decode (pa_decode_shared_prefix) against
the fp64 oracle, on fork families built through the oracle block manager.

The oracle attends over each sequence's own tokens through its own table;
the library reads each group's common prefix once for all members and merges
it with each member's remaining tokens, so the two must agree to 2e-3
(fp16/bf16) whatever the grouping, the partition length, the group size
(several member tiles) and the prefix/suffix split (including members with
no suffix).  The groups and prefixes come from the oracle's prefix_groups.
"""
import os

import numpy as np
import torch  # noqa: F401  (first import can be slow on a fresh box; keep it out of test timeouts)
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_families, run_shared_prefix, out_to_f64, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def _want(case, dtype):
    return paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], dtype)


# (prompt tokens, appended tokens per member); member 0 is the prompt's own sequence
FAMILIES = [(100, [0, 7, 50, 3]), (37, [5, 1]), (64, [0, 10]), (20, [4])]


@pytest.mark.parametrize("dtype,kv_heads,group,head_dim,bs", [
    ("f16", 2, 1, 128, 16), ("bf16", 2, 1, 128, 16), ("f16", 1, 8, 128, 32), ("bf16", 2, 4, 64, 16),
    ("bf16", 1, 2, 128, 64)])
@pytest.mark.parametrize("partition", [0, 32, 64, 256])
def test_shared_prefix_matches_oracle(gpu, dtype, kv_heads, group, head_dim, bs, partition):
    pk = gpu
    if partition % bs:
        pytest.skip("partition is not a multiple of the block size")
    case = build_families(FAMILIES, kv_heads, group, head_dim, bs, dtype, seed=11 + bs + group)
    assert case["prefix"].max() > 0
    got = out_to_f64(run_shared_prefix(pk, case, kv_heads, head_dim, bs, dtype, out_dtype="f32",
                                       partition_tokens=partition))
    assert np.max(np.abs(got - _want(case, dtype))) <= TOL[dtype]


@pytest.mark.parametrize("group", [1, 8])
def test_large_groups_span_member_tiles(gpu, group):
    """20 samples of one prompt (2 tiles at G=1, 10 at G=8) plus a second family."""
    pk = gpu
    fam = [(90, [0] + [int(x) for x in np.random.default_rng(5).integers(0, 40, size=19)]), (33, [2, 9, 0])]
    case = build_families(fam, 1, group, 128, 16, "f16", seed=21)
    assert case["max_group"] == 20
    got = out_to_f64(run_shared_prefix(pk, case, 1, 128, 16, "f16", out_dtype="f32"))
    assert np.max(np.abs(got - _want(case, "f16"))) <= TOL["f16"]


def test_same_result_as_plain_decode_and_no_groups(gpu):
    """The plain decode and the shared-prefix call with its grouping removed
    (one group of one per sequence, no prefixes) agree with the oracle too."""
    import torch
    pk = gpu
    case = build_families(FAMILIES, 2, 2, 128, 16, "bf16", seed=3)
    want = _want(case, "bf16")
    shared = out_to_f64(run_shared_prefix(pk, case, 2, 128, 16, "bf16", out_dtype="f32"))
    n = len(case["ids"])
    alone = out_to_f64(run_shared_prefix(pk, case, 2, 128, 16, "bf16", out_dtype="f32",
                                         group_start=np.arange(n + 1), prefix=np.zeros(n, dtype=np.int32),
                                         max_prefix=16))
    pool = pk.Pool(case["num_blocks"], 16, 2, 128, "bf16",
                   k=torch.from_numpy(case["k_pool"].view(np.int16)).view(torch.bfloat16).cuda(),
                   v=torch.from_numpy(case["v_pool"].view(np.int16)).view(torch.bfloat16).cuda())
    plain = out_to_f64(pk.decode(pool, torch.from_numpy(case["q"].view(np.int16)).view(torch.bfloat16).cuda(),
                                 torch.from_numpy(case["tables"]).cuda(), torch.from_numpy(case["lens"]).cuda(),
                                 int(case["lens"].max()), out_dtype="f32"))
    for got in (shared, alone, plain):
        assert np.max(np.abs(got - want)) <= TOL["bf16"]


def test_fp32_pool_takes_the_plain_path(gpu):
    pk = gpu
    case = build_families(FAMILIES, 1, 4, 64, 16, "f32", seed=9)
    got = out_to_f64(run_shared_prefix(pk, case, 1, 64, 16, "f32"))
    assert np.max(np.abs(got - _want(case, "f32"))) <= TOL["f32"]


def test_bad_prefix_block_marks_the_whole_group(gpu):
    """With host validation off, a block id outside the pool inside a shared
    prefix gives NaN rows for that group's members only."""
    pk = gpu
    case = build_families(FAMILIES, 1, 1, 128, 16, "f16", seed=4)
    want = _want(case, "f16")
    gs, pre = case["group_start"], case["prefix"]
    k = int(np.argmax(pre))                        # a member of the first group with a prefix
    g = int(np.searchsorted(gs, k, side="right")) - 1
    members = list(range(gs[g], gs[g + 1]))
    case["tables"][gs[g], 0] = 1 << 30             # the prefix is read through the group's first table
    os.environ["PA_DEBUG_VALIDATE"] = "0"
    try:
        got = out_to_f64(run_shared_prefix(pk, case, 1, 128, 16, "f16", out_dtype="f32"))
    finally:
        os.environ["PA_DEBUG_VALIDATE"] = "1"
    others = [i for i in range(len(case["ids"])) if i not in members]
    assert np.all(np.isnan(got[members]))
    assert np.max(np.abs(got[others] - want[others])) <= TOL["f16"]


@pytest.mark.parametrize("breakage", ["unequal", "unaligned", "too_long", "other_blocks", "group_start"])
def test_validation_rejects_a_broken_grouping(gpu, breakage):
    pk = gpu
    case = build_families(FAMILIES, 1, 1, 128, 16, "f16", seed=6)
    gs, pre = case["group_start"].copy(), case["prefix"].copy()
    first = int(np.argmax(pre))
    g = int(np.searchsorted(gs, first, side="right")) - 1
    a, b = int(gs[g]), int(gs[g + 1])
    if breakage == "unequal":
        pre[b - 1] -= 16
    elif breakage == "unaligned":
        pre[a:b] -= 1
    elif breakage == "too_long":
        pre[a:b] = int(case["lens"][a:b].min()) + 16
    elif breakage == "other_blocks":
        case["tables"][b - 1, 0] = (int(case["tables"][a, 0]) + 1) % case["num_blocks"]
    else:
        gs[1] += 1
    with pytest.raises(pk.PaError):
        run_shared_prefix(pk, case, 1, 128, 16, "f16", group_start=gs, prefix=pre,
                          max_prefix=int(case["lens"].max()))
