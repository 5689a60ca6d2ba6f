"""Seeded random decode cases across the whole supported space, against the
fp64 oracle.

The parametrised tests walk grids of one or two dimensions at a time; these
cases cross all of them at once: pool dtype, head_dim, block_size, group
size, kv-head counts that are not powers of two, ragged batches with empty,
one-token and block-boundary lengths, every split mode (automatic, fixed
partitions of a random number of blocks, uniform, balanced), the output in
the pool dtype or fp32, the default or a custom logit scale, and plain
decode or pa_decode_append.  Pools are NaN-poisoned outside live tokens.

Tolerance: 1e-5 (fp32 pools) or 2e-3 (fp16/bf16), plus half an output ulp
when the output is rounded to a 16-bit type (round to nearest even).
"""
import os

import numpy as np
import pytest

from oracle.attention import paged_decode
from tests.gpu_util import build_case, to_torch, to_bits, out_to_f64, NAN_BITS, TOL

pytestmark = pytest.mark.gpu

N_CASES = 200
OUT_HALF_ULP = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}   # relative, round to nearest


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    import paged_kv_cache_355_amd as pk
    pk.lib()
    yield pk


def draw_case(i):
    rng = np.random.default_rng(70000 + i)
    dtype = ["f32", "f16", "bf16"][rng.integers(3)]
    head_dim = [64, 128][rng.integers(2)]
    bs = [4, 8, 16, 32, 64][rng.integers(5)]
    group = [1, 2, 4, 8][rng.integers(4)]
    kv_heads = [1, 2, 3, 5][rng.integers(4)]
    B = int(rng.integers(1, 13))
    special = [0, 1, bs - 1, bs, bs + 1, 16 * bs + 3]
    lens = [int(special[rng.integers(len(special))]) if rng.random() < 0.4 else int(rng.integers(1, 3000))
            for _ in range(B)]
    mode = ["auto", "fixed", "uniform", "balanced"][rng.integers(4)]
    out_dtype = dtype if rng.random() < 0.5 else "f32"
    scale = None if rng.random() < 0.5 else float(rng.uniform(0.02, 0.2))
    append = bool(rng.random() < 0.3)
    part_blocks = int(rng.integers(1, 40))
    return dict(dtype=dtype, head_dim=head_dim, bs=bs, group=group, kv_heads=kv_heads, lens=lens, mode=mode,
                out_dtype=out_dtype, scale=scale, append=append, part_blocks=part_blocks, seed=71000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(gpu, i):
    import torch
    pk = gpu
    c = draw_case(i)
    print(f"[fuzz {i}] {c}", flush=True)
    dtype, d, bs, G, hkv = c["dtype"], c["head_dim"], c["bs"], c["group"], c["kv_heads"]
    case = build_case(c["lens"], hkv, G, d, bs, dtype, c["seed"], scale=d ** -0.5)
    part = {"auto": 0, "fixed": c["part_blocks"] * bs, "uniform": pk.PA_PARTITION_UNIFORM,
            "balanced": pk.PA_PARTITION_BALANCED}[c["mode"]]
    k_pool, v_pool = case["k_pool"], case["v_pool"]
    append = None
    if c["append"]:
        # the last token of every non-empty sequence arrives as the new token
        B = len(c["lens"])
        k_new = np.zeros((B, hkv, d), dtype=k_pool.dtype)
        v_new = np.zeros_like(k_new)
        slots = np.full(B, -1, dtype=np.int32)
        k_pool, v_pool = k_pool.copy(), v_pool.copy()
        for s, n in enumerate(c["lens"]):
            if n == 0:
                continue
            slot = case["bm"].token_slots(s)[n - 1]
            b, o = divmod(slot, bs)
            slots[s] = slot
            k_new[s], v_new[s] = case["k_pool"][b, :, o, :], case["v_pool"][b, :, o, :]
            k_pool[b, :, o, :] = NAN_BITS[dtype]
            v_pool[b, :, o, :] = NAN_BITS[dtype]
        append = (to_torch(k_new, dtype), to_torch(v_new, dtype), torch.from_numpy(slots).cuda())
    pool = pk.Pool(case["num_blocks"], bs, hkv, d, dtype, k=to_torch(k_pool, dtype), v=to_torch(v_pool, dtype))
    out = pk.decode(pool, to_torch(case["q"], dtype), torch.from_numpy(case["tables"]).cuda(),
                    torch.from_numpy(case["lens"]).cuda(), int(max(case["lens"].max(), 0)),
                    out_dtype=c["out_dtype"], scale=c["scale"], partition_tokens=part, append=append)
    torch.cuda.synchronize()
    if c["append"]:
        assert np.array_equal(to_bits(pool.k, dtype), case["k_pool"])
        assert np.array_equal(to_bits(pool.v, dtype), case["v_pool"])
    want = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], dtype,
                        scale=c["scale"])
    got = out_to_f64(out)
    assert np.all(np.isfinite(got))
    tol = TOL[dtype] + np.abs(want) * OUT_HALF_ULP[c["out_dtype"]]
    excess = float(np.max(np.abs(got - want) - tol))
    print(f"[fuzz {i}] max |err| {float(np.max(np.abs(got - want))):.3e}", flush=True)
    assert excess <= 0.0
    for s, n in enumerate(c["lens"]):
        if n == 0:
            assert np.all(got[s] == 0.0)


N_FAMILY_CASES = 64


def draw_families(i):
    rng = np.random.default_rng(80000 + i)
    dtype = ["f32", "f16", "bf16"][rng.integers(3)] if rng.random() < 0.2 else ["f16", "bf16"][rng.integers(2)]
    bs = [4, 16, 32, 64][rng.integers(4)] if rng.random() < 0.25 else [16, 32][rng.integers(2)]
    group = [1, 2, 4, 8][rng.integers(4)]
    kv_heads = [1, 2, 3][rng.integers(3)]
    head_dim = [64, 128][rng.integers(2)]
    fams = []
    for _ in range(int(rng.integers(1, 6))):
        prompt = int(rng.integers(1, 700)) if rng.random() < 0.8 else int(rng.integers(1, 8)) * bs
        members = int(rng.integers(1, 21))
        fams.append((prompt, [int(x) for x in rng.integers(0, 120, size=members)]))
    part = 0 if rng.random() < 0.5 else int(rng.integers(1, 20)) * bs
    return dict(dtype=dtype, bs=bs, group=group, kv_heads=kv_heads, head_dim=head_dim, families=fams,
                partition=part, seed=81000 + i)


@pytest.mark.parametrize("i", range(N_FAMILY_CASES))
def test_random_forked_batch_through_shared_prefix_decode(gpu, i):
    """Random fork families (prompts of any length, 1-20 members, 0-119
    appended tokens each, so copy-on-write at part-filled shared blocks) in the
    oracle's dispatch order and prefix groups, through pa_decode_shared_prefix
    (fp32 pools and blocks under 16 tokens take the plain decode inside)."""
    from tests.gpu_util import build_families, run_shared_prefix
    pk = gpu
    c = draw_families(i)
    print(f"[family fuzz {i}] {c}", flush=True)
    case = build_families(c["families"], c["kv_heads"], c["group"], c["head_dim"], c["bs"], c["dtype"], c["seed"],
                          scale=c["head_dim"] ** -0.5)
    got = out_to_f64(run_shared_prefix(pk, case, c["kv_heads"], c["head_dim"], c["bs"], c["dtype"], out_dtype="f32",
                                       partition_tokens=c["partition"]))
    want = paged_decode(case["q"], case["k_pool"], case["v_pool"], case["tables"], case["lens"], c["dtype"])
    err = float(np.max(np.abs(got - want)))
    print(f"[family fuzz {i}] groups {len(case['group_start']) - 1}, max prefix {int(case['prefix'].max())}, "
          f"max |err| {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err <= TOL[c["dtype"]]
