"""Pins for oracle.attention (paged decode in float64).

Each test fixes the oracle by something other than itself:

* a library special case — torch's scaled_dot_product_attention in float64 on
  the CPU, on contiguous K/V laid out in an identity block table ([P2 §1.1]);
* brute force — pure-Python loops with math.exp over the logical (never paged)
  K/V arrays, on tiny inputs;
* closed forms — one token, zero query, equal keys, a dominant key, per-head
  constant values (pins the GQA mapping);
* invariants — physical placement, shared vs private prefix blocks, padding
  contents, logical token order.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.attention import paged_decode, gather_sequence
from oracle.numerics import F32, F16, BF16, to_f64
from oracle.block_manager import OracleBlockManager
from oracle.kv_ops import write_kv
from workloads import round_to_bits


def _pool(nb, hkv, bs, d, dtype, fill=np.nan):
    bits = round_to_bits(np.full((nb, hkv, bs, d), fill, dtype=np.float32), dtype)
    return bits, bits.copy()


def _place(lengths, hkv, d, bs, dtype, rng, free_order=None, scale=1.0):
    """Write random logical K/V per sequence into a paged pool.

    Returns (k_pool, v_pool, tables, logical_k, logical_v) where logical_* are
    the per-sequence [hkv][L][d] bit arrays as drawn, before paging.
    """
    nb = sum(-(-n // bs) for n in lengths) + 3
    order = list(range(nb)) if free_order is None else list(free_order)
    bm = OracleBlockManager(nb, bs, order)
    kp, vp = _pool(nb, hkv, bs, d, dtype)
    lk, lv, tables = [], [], []
    for s, n in enumerate(lengths):
        bm.add_seq(s, n)
        k = round_to_bits(rng.standard_normal((n, hkv, d)).astype(np.float32) * scale, dtype)
        v = round_to_bits(rng.standard_normal((n, hkv, d)).astype(np.float32) * scale, dtype)
        write_kv(kp, vp, k, v, bm.token_slots(s))
        lk.append(k.transpose(1, 0, 2))
        lv.append(v.transpose(1, 0, 2))
        tables.append(bm.block_table(s)[0])
    stride = max([len(t) for t in tables] + [1])
    tables = [t + [-1] * (stride - len(t)) for t in tables]
    return kp, vp, tables, lk, lv


def test_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    B, hq, hkv, d, bs = 3, 6, 2, 16, 4
    lengths = [9, 1, 14]
    kp, vp, tables, lk, lv = _place(lengths, hkv, d, bs, F32, rng)
    q = round_to_bits(rng.standard_normal((B, hq, d)).astype(np.float32), F32)
    got = paged_decode(q, kp, vp, tables, lengths, F32)
    qf = to_f64(q, F32)
    G = hq // hkv
    for s, n in enumerate(lengths):
        k = torch.from_numpy(to_f64(lk[s], F32)).repeat_interleave(G, dim=0)   # [hq][n][d]
        v = torch.from_numpy(to_f64(lv[s], F32)).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(qf[s]).unsqueeze(1)                                # [hq][1][d]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v).squeeze(1).numpy()
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-13)


def _brute(q, K, V, scale):
    """Pure-Python softmax attention for one query row over rows of K/V."""
    logits = [scale * sum(qi * ki for qi, ki in zip(q, krow)) for krow in K]
    top = max(logits)
    w = [math.exp(z - top) for z in logits]
    tot = sum(w)
    return [sum(w[t] * V[t][j] for t in range(len(K))) / tot for j in range(len(q))]


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_matches_brute_force_on_logical_arrays(data):
    B = data.draw(st.integers(1, 3))
    hkv = data.draw(st.integers(1, 2))
    G = data.draw(st.sampled_from([1, 2, 3]))
    d = data.draw(st.integers(1, 6))
    bs = data.draw(st.sampled_from([1, 2, 4]))
    dtype = data.draw(st.sampled_from([F32, F16, BF16]))
    lengths = data.draw(st.lists(st.integers(0, 21), min_size=B, max_size=B))
    seed = data.draw(st.integers(0, 2 ** 31))
    rng = np.random.default_rng(seed)
    nb = sum(-(-n // bs) for n in lengths) + 3
    order = list(rng.permutation(nb))
    kp, vp, tables, lk, lv = _place(lengths, hkv, d, bs, dtype, rng, order)
    hq = hkv * G
    q = round_to_bits(rng.standard_normal((B, hq, d)).astype(np.float32), dtype)
    scale = data.draw(st.sampled_from([None, 0.37]))
    got = paged_decode(q, kp, vp, tables, lengths, dtype, scale=scale)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    qf = to_f64(q, dtype)
    for s, n in enumerate(lengths):
        for h in range(hq):
            if n == 0:
                assert np.all(got[s, h] == 0.0)
                continue
            K = to_f64(lk[s][h // G], dtype).tolist()
            V = to_f64(lv[s][h // G], dtype).tolist()
            ref = _brute(qf[s, h].tolist(), K, V, sc)
            np.testing.assert_allclose(got[s, h], ref, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(2)
    kp, vp, tables, lk, lv = _place([1], 1, 8, 4, F16, rng)
    q = round_to_bits(rng.standard_normal((1, 1, 8)).astype(np.float32), F16)
    got = paged_decode(q, kp, vp, tables, [1], F16)
    assert np.array_equal(got[0, 0], to_f64(lv[0][0][0], F16))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    kp, vp, tables, lk, lv = _place([13], 1, 8, 4, F32, rng)
    q = np.zeros((1, 1, 8), dtype=np.uint32)
    got = paged_decode(q, kp, vp, tables, [13], F32)
    np.testing.assert_allclose(got[0, 0], to_f64(lv[0][0], F32).mean(axis=0), rtol=0, atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    bs, d, n = 4, 8, 11
    bm = OracleBlockManager(8, bs)
    bm.add_seq(0, n)
    kp, vp = _pool(8, 1, bs, d, BF16)
    krow = round_to_bits(rng.standard_normal((1, 1, d)).astype(np.float32), BF16)
    v = round_to_bits(rng.standard_normal((n, 1, d)).astype(np.float32), BF16)
    write_kv(kp, vp, np.repeat(krow, n, axis=0), v, bm.token_slots(0))
    q = round_to_bits(rng.standard_normal((1, 1, d)).astype(np.float32), BF16)
    got = paged_decode(q, kp, vp, [bm.block_table(0)[0]], [n], BF16)
    np.testing.assert_allclose(got[0, 0], to_f64(v, BF16)[:, 0].mean(axis=0), rtol=0, atol=1e-15)


def test_dominant_key_selects_its_value():
    """Logit gap Δ ≥ 60 → the output is V_j within (n-1)·e^{-Δ}·max|V|."""
    rng = np.random.default_rng(5)
    d, n, j = 16, 9, 6
    kp, vp, tables, lk, lv = _place([n], 1, d, 4, F32, rng, scale=0.1)
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 40.0
    # make key j = 10·e0 (logit 100) and every other key orthogonal to q
    bm_slots = [tables[0][t // 4] * 4 + t % 4 for t in range(n)]
    kf = kp.view(np.float32)
    for t in range(n):
        b, o = divmod(bm_slots[t], 4)
        kf[b, 0, o, 0] = 10.0 if t == j else 0.0
    got = paged_decode(q.view(np.uint32), kp, vp, tables, [n], F32, scale=0.25)
    want = to_f64(lv[0][0][j], F32)
    assert np.max(np.abs(got[0, 0] - want)) <= (n - 1) * math.exp(-100.0) * 10


def test_gqa_mapping_consecutive_heads_share_a_kv_head():
    rng = np.random.default_rng(6)
    hkv, G, d, bs, n = 4, 3, 8, 4, 10
    bm = OracleBlockManager(8, bs)
    bm.add_seq(0, n)
    kp, vp = _pool(8, hkv, bs, d, F32)
    k = round_to_bits(rng.standard_normal((n, hkv, d)).astype(np.float32), F32)
    v = round_to_bits(np.broadcast_to(np.arange(1, hkv + 1, dtype=np.float32)[None, :, None], (n, hkv, d)), F32)
    write_kv(kp, vp, k, v, bm.token_slots(0))
    q = round_to_bits(rng.standard_normal((1, hkv * G, d)).astype(np.float32), F32)
    got = paged_decode(q, kp, vp, [bm.block_table(0)[0]], [n], F32)
    for h in range(hkv * G):
        np.testing.assert_allclose(got[0, h], h // G + 1, rtol=1e-14)


def test_placement_permutation_is_bit_identical():
    lengths = [7, 18, 3]
    outs = []
    for seed in range(4):
        rng = np.random.default_rng(99)          # same values every time
        perm = np.random.default_rng(seed).permutation(sum(-(-n // 4) for n in lengths) + 3)
        kp, vp, tables, _, _ = _place(lengths, 2, 8, 4, F16, rng, perm)
        q = round_to_bits(np.random.default_rng(7).standard_normal((3, 4, 8)).astype(np.float32), F16)
        outs.append(paged_decode(q, kp, vp, tables, lengths, F16))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_shared_prefix_equals_private_copies():
    rng = np.random.default_rng(8)
    bs, d, hkv, n0 = 4, 8, 2, 10
    bm = OracleBlockManager(32, bs)
    bm.add_seq(0, n0)
    bm.fork(0, 1)
    kp, vp = _pool(32, hkv, bs, d, F16)
    k = round_to_bits(rng.standard_normal((n0, hkv, d)).astype(np.float32), F16)
    v = round_to_bits(rng.standard_normal((n0, hkv, d)).astype(np.float32), F16)
    write_kv(kp, vp, k, v, bm.token_slots(0))
    # private copy of the same bytes under another sequence
    bm.add_seq(2, n0)
    write_kv(kp, vp, k, v, bm.token_slots(2))
    q = round_to_bits(rng.standard_normal((1, hkv, d)).astype(np.float32), F16)
    q3 = np.repeat(q, 3, axis=0)
    tables = bm.padded_tables([0, 1, 2], 3)
    got = paged_decode(q3, kp, vp, tables, [n0] * 3, F16)
    assert tables[0] == tables[1] and set(tables[0]).isdisjoint(tables[2])
    assert np.array_equal(got[0], got[1]) and np.array_equal(got[0], got[2])


def test_padding_contents_are_never_read():
    rng = np.random.default_rng(9)
    lengths = [5, 9]
    kp, vp, tables, _, _ = _place(lengths, 1, 8, 4, F32, rng)   # padding is NaN
    q = round_to_bits(rng.standard_normal((2, 1, 8)).astype(np.float32), F32)
    got = paged_decode(q, kp, vp, tables, lengths, F32)
    assert np.all(np.isfinite(got))
    kp2 = kp.copy()
    kp2[kp2.view(np.float32) != kp2.view(np.float32)] = 0      # NaN → 0
    assert np.array_equal(paged_decode(q, kp2, vp, tables, lengths, F32), got)


def test_logical_order_permutation_changes_only_rounding():
    rng = np.random.default_rng(10)
    n, d = 23, 8
    kp, vp, tables, lk, lv = _place([n], 1, d, 4, F32, rng)
    q = round_to_bits(rng.standard_normal((1, 1, d)).astype(np.float32), F32)
    base = paged_decode(q, kp, vp, tables, [n], F32)
    perm = rng.permutation(n)
    kp2, vp2 = kp.copy(), vp.copy()
    slots = [tables[0][t // 4] * 4 + t % 4 for t in range(n)]
    write_kv(kp2, vp2, lk[0].transpose(1, 0, 2)[perm], lv[0].transpose(1, 0, 2)[perm], slots)
    np.testing.assert_allclose(paged_decode(q, kp2, vp2, tables, [n], F32), base, rtol=1e-13, atol=1e-15)


def test_gather_follows_the_table():
    pool = np.arange(5 * 1 * 2 * 1).reshape(5, 1, 2, 1)
    got = gather_sequence(pool, [3, 0, 4], 5, 2)
    assert got[0, :, 0].tolist() == [6, 7, 0, 1, 8]
