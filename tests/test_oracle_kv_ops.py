"""Pins for oracle.kv_ops: slot-mapped KV write and copy-on-write block copy.

Expected pool contents are built independently of the oracle's indexing: the
tests address the pool with explicit (block, head, offset) loops and compare
whole pools bit for bit, including every untouched byte.
"""
import numpy as np
import pytest

from oracle.kv_ops import write_kv, copy_blocks


def _pool(nb=6, hkv=2, bs=4, d=3, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint16)
    return k, v


def test_write_lands_in_slot_and_nowhere_else():
    k, v = _pool()
    k0, v0 = k.copy(), v.copy()
    rng = np.random.default_rng(1)
    kn = rng.integers(0, 2 ** 16, size=(3, 2, 3), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, size=(3, 2, 3), dtype=np.uint16)
    slots = [9, -1, 22]                   # (block 2, off 1), skipped, (block 5, off 2)
    write_kv(k, v, kn, vn, slots)
    want_k, want_v = k0.copy(), v0.copy()
    for i, (b, o) in {0: (2, 1), 2: (5, 2)}.items():
        for h in range(2):
            for j in range(3):
                want_k[b, h, o, j] = kn[i, h, j]
                want_v[b, h, o, j] = vn[i, h, j]
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)


def test_write_preserves_nan_payload_bits():
    k = np.zeros((2, 1, 2, 2), dtype=np.uint32)
    v = np.zeros_like(k)
    payload = np.array([[[0x7FC00001, 0xFFFFFFFF]]], dtype=np.uint32)
    write_kv(k, v, payload, payload, [3])
    assert k[1, 0, 1].tolist() == [0x7FC00001, 0xFFFFFFFF]


def test_write_rejects_duplicate_slots_and_out_of_range():
    k, v = _pool()
    row = np.zeros((2, 2, 3), dtype=np.uint16)
    with pytest.raises(ValueError):
        write_kv(k, v, row, row, [5, 5])
    with pytest.raises(IndexError):
        write_kv(k, v, row[:1], row[:1], [6 * 4])


def test_copy_is_simultaneous_and_whole_block():
    k, v = _pool()
    k0, v0 = k.copy(), v.copy()
    copy_blocks(k, v, [(1, 4), (0, 3)])
    want_k, want_v = k0.copy(), v0.copy()
    want_k[4], want_v[4] = k0[1], v0[1]
    want_k[3], want_v[3] = k0[0], v0[0]
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)


def test_copy_same_source_twice():
    k, v = _pool()
    k0 = k.copy()
    copy_blocks(k, v, [(2, 0), (2, 5)])
    assert np.array_equal(k[0], k0[2]) and np.array_equal(k[5], k0[2])
    assert np.array_equal(k[1], k0[1])


def test_copy_rejects_aliasing():
    k, v = _pool()
    with pytest.raises(ValueError):
        copy_blocks(k, v, [(0, 1), (2, 1)])
    with pytest.raises(ValueError):
        copy_blocks(k, v, [(0, 1), (1, 2)])
    with pytest.raises(IndexError):
        copy_blocks(k, v, [(0, 6)])


def test_copy_empty_is_noop():
    k, v = _pool()
    k0 = k.copy()
    copy_blocks(k, v, [])
    assert np.array_equal(k, k0)


def test_swap_out_layout_and_round_trip():
    """Every element tagged with (block, head, slot, dim) in K and the same
    plus an offset in V: swap_out returns [n][K, V] tiles in the order asked,
    and swap_in writes them back into other blocks unchanged."""
    from oracle.kv_ops import swap_out, swap_in
    nb, hkv, bs, d = 6, 2, 4, 3
    idx = np.arange(nb * hkv * bs * d, dtype=np.uint32).reshape(nb, hkv, bs, d)
    k, v = idx.copy(), idx + np.uint32(1 << 20)
    host = swap_out(k, v, [4, 1])
    assert host.shape == (2, 2, hkv, bs, d)
    assert np.array_equal(host[0, 0], idx[4]) and np.array_equal(host[1, 1], idx[1] + (1 << 20))
    k2, v2 = np.zeros_like(k), np.zeros_like(v)
    swap_in(k2, v2, [0, 5], host)
    assert np.array_equal(k2[0], k[4]) and np.array_equal(v2[5], v[1])
    assert not k2[1:5].any() and not v2[1:5].any()
    with pytest.raises(ValueError):
        swap_in(k2, v2, [2, 2], host)
