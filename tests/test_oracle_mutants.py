"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU, via
monkeypatch) and checks that at least one pin test then fails.  A pin set that
passes a mutant would not have caught that mistake in the oracle itself.
"""
import math

import numpy as np
import pytest

import oracle.attention as att
import oracle.block_manager as bmmod
from oracle.numerics import to_f64
import tests.test_oracle_attention as ta
import tests.test_oracle_block_manager as tb

ATTENTION_PINS = [
    ta.test_matches_torch_sdpa_float64,
    ta.test_single_token_returns_its_value_exactly,
    ta.test_zero_query_gives_mean_of_values,
    ta.test_dominant_key_selects_its_value,
    ta.test_gqa_mapping_consecutive_heads_share_a_kv_head,
    ta.test_gather_follows_the_table,
    ta.test_padding_contents_are_never_read,
]


def _fails(pins, *args):
    for pin in pins:
        try:
            pin(*args)
        except Exception:
            return True
    return False


def _softmax_no_scale(q, keys, values, scale):
    logits = keys @ q
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ values


def _softmax_scale_by_sqrt(q, keys, values, scale):
    logits = (keys @ q) / scale
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ values


def _softmax_unnormalised(q, keys, values, scale):
    logits = (keys @ q) * scale
    return np.exp(logits - logits.max()) @ values


def _softmax_wrong_sign(q, keys, values, scale):
    logits = -(keys @ q) * scale
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ values


def _softmax_keys_as_values(q, keys, values, scale):
    logits = (keys @ q) * scale
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ keys


def _gather_off_by_one(pool, table, length, block_size):
    nb, hkv, bs, d = pool.shape
    out = np.empty((hkv, length, d), dtype=pool.dtype)
    for t in range(length):
        out[:, t, :] = pool[int(table[t // block_size]), :, (t + 1) % block_size, :]
    return out


def _gather_logical_index(pool, table, length, block_size):
    nb, hkv, bs, d = pool.shape
    out = np.empty((hkv, length, d), dtype=pool.dtype)
    for t in range(length):
        out[:, t, :] = pool[t // block_size, :, t % block_size, :]     # table ignored
    return out


@pytest.mark.parametrize("name,mutant", [
    ("no scale", _softmax_no_scale),
    ("scale inverted", _softmax_scale_by_sqrt),
    ("no normalisation", _softmax_unnormalised),
    ("logit sign", _softmax_wrong_sign),
    ("K used as V", _softmax_keys_as_values),
])
def test_softmax_mutants_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(att, "softmax_attend", mutant)
    assert _fails(ATTENTION_PINS), name


@pytest.mark.parametrize("name,mutant", [
    ("offset off by one", _gather_off_by_one),
    ("block table ignored", _gather_logical_index),
])
def test_gather_mutants_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(att, "gather_sequence", mutant)
    assert _fails(ATTENTION_PINS), name


def test_gqa_mapping_mutant_is_caught(monkeypatch):
    original = att.paged_decode

    def modulo_mapping(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens, dtype,
                       scale=None, q_dtype=None):
        # query head h reads kv-head h mod Hkv instead of ⌊h/G⌋
        nb, hkv, bs, d = k_pool_bits.shape
        B, hq, _ = q_bits.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        qf = to_f64(q_bits, q_dtype or dtype)
        out = np.zeros((B, hq, d))
        for s in range(B):
            n = int(context_lens[s])
            if n == 0:
                continue
            k = to_f64(att.gather_sequence(k_pool_bits, block_tables[s], n, bs), dtype)
            v = to_f64(att.gather_sequence(v_pool_bits, block_tables[s], n, bs), dtype)
            for h in range(hq):
                out[s, h] = att.softmax_attend(qf[s, h], k[h % hkv], v[h % hkv], scale)
        return out

    monkeypatch.setattr(ta, "paged_decode", modulo_mapping)
    assert _fails([ta.test_gqa_mapping_consecutive_heads_share_a_kv_head,
                   ta.test_matches_torch_sdpa_float64])
    monkeypatch.setattr(ta, "paged_decode", original)


BM_PINS = [
    tb.test_worked_example_appends,
    tb.test_copy_on_write_tie_break,
    tb.test_full_shared_block_needs_no_copy,
    tb.test_free_returns_blocks_fifo,
    tb.test_pool_exhaustion_leaves_state_unchanged,
    tb.test_exhaustion_counts_in_batch_copies,
]


class _LifoFree(bmmod.OracleBlockManager):
    def free_seq(self, seq_id):
        seq = self.seqs.pop(seq_id)
        for b in seq.table:
            self.rc[b] -= 1
            if self.rc[b] == 0:
                self.free.appendleft(b)


class _AlwaysCopy(bmmod.OracleBlockManager):
    """Copies a part-filled last block even when nobody else holds it."""

    def append_slot(self, seq_id):
        seq = self.seqs[seq_id]
        t, bs = seq.length, self.block_size
        src = dst = -1
        if t % bs == 0:
            seq.table.append(self._pop_free())
        else:
            old, new = seq.table[-1], self._pop_free()
            self.rc[old] -= 1
            if self.rc[old] == 0:
                self.free.append(old)
            seq.table[-1] = new
            src, dst = old, new
        seq.length = t + 1
        return seq.table[t // bs] * bs + t % bs, src, dst


class _NoCopy(bmmod.OracleBlockManager):
    def append_slot(self, seq_id):
        seq = self.seqs[seq_id]
        t, bs = seq.length, self.block_size
        if t % bs == 0:
            seq.table.append(self._pop_free())
        seq.length = t + 1
        return seq.table[t // bs] * bs + t % bs, -1, -1


class _CopyAfterDecrementOrder(bmmod.OracleBlockManager):
    """Copies iff rc > 2: leaves two writers on one block."""

    def append_slot(self, seq_id):
        seq = self.seqs[seq_id]
        t, bs = seq.length, self.block_size
        src = dst = -1
        if t % bs == 0:
            seq.table.append(self._pop_free())
        elif self.rc[seq.table[-1]] > 2:
            old, new = seq.table[-1], self._pop_free()
            self.rc[old] -= 1
            seq.table[-1] = new
            src, dst = old, new
        seq.length = t + 1
        return seq.table[t // bs] * bs + t % bs, src, dst


@pytest.mark.parametrize("name,cls", [
    ("LIFO release", _LifoFree),
    ("copy even when unshared", _AlwaysCopy),
    ("never copy", _NoCopy),
    ("copy threshold off by one", _CopyAfterDecrementOrder),
])
def test_block_manager_mutants_are_caught(monkeypatch, name, cls):
    monkeypatch.setattr(tb, "OracleBlockManager", cls)
    assert _fails(BM_PINS), name
