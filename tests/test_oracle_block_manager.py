"""Pins for oracle.block_manager and oracle.accounting.

* The pages' worked example ([P1] "Paged Attention 的工作原理" / "块表") is a
  literal fixture in tests/golden/worked_example.json.
* The decode-step procedure ([P2 §3.2.2]), the free list ([P2 §3.3]) and
  copy-on-write ([P2 §3.4]) are pinned by hand-traced small cases whose
  expected tables/slots are written out by hand below.
* A hypothesis state machine checks the invariants the pages imply for any
  call sequence.
* dispatch_order (a scheduling choice, not the pages') is pinned by a
  hand-ordered batch, by its reduction to a plain stable sort when nothing is
  shared, and by the properties any such order must have.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.stateful import RuleBasedStateMachine, rule, invariant, precondition

from oracle.block_manager import OracleBlockManager, NoBlocksError
from oracle import accounting


@pytest.fixture
def example(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_table_and_placement(example):
    bs = example["block_size"]
    table = example["block_table"]
    nb = 16
    order = table + [b for b in range(nb) if b not in table]
    bm = OracleBlockManager(nb, bs, order)
    bm.add_seq(0, example["num_tokens"])
    got_table, n = bm.block_table(0)
    assert got_table == table and n == example["num_tokens"]
    slots = bm.token_slots(0)
    # every printed token sits in the printed block at its printed position
    for j, toks in enumerate(example["tokens_per_block"]):
        for pos, tok in enumerate(toks):
            assert slots[tok] // bs == table[j]
            assert slots[tok] % bs == pos
    st_ = bm.stats()
    assert st_["used_blocks"] * bs - st_["filled_slots"] == example["empty_slots_last_block"]


def test_worked_example_waste(example):
    reserved, used = accounting.contiguous_slots([example["num_tokens"]], example["contiguous_reserved_slots"])
    assert (reserved, used) == (example["contiguous_reserved_slots"], example["contiguous_used_slots"])
    assert reserved - used == example["contiguous_wasted_slots"]
    assert [reserved - used, reserved] == example["contiguous_waste"]
    p_reserved, p_used = accounting.paged_slots([example["num_tokens"]], example["block_size"])
    assert [p_reserved - p_used, example["block_size"]] == example["paged_last_block_waste"]


def test_worked_example_appends():
    """Hand-traced continuation of the example (bs 4, free order 5,12,3,9,0,...)."""
    order = [5, 12, 3, 9, 0, 1, 2, 4, 6, 7, 8, 10, 11, 13, 14, 15]
    bm = OracleBlockManager(16, 4, order)
    bm.add_seq(0, 10)                     # blocks 5, 12, 3
    bm.add_seq(1, 7)                      # blocks 9, 0
    assert bm.block_table(1) == ([9, 0], 7)
    assert bm.token_slots(1) == [36, 37, 38, 39, 0, 1, 2]
    slots, pairs = bm.step([0, 1])        # token 10 → block 3 offset 2; token 7 → block 0 offset 3
    assert slots == [14, 3] and pairs == []
    slots, _ = bm.step([0, 1])            # token 11 → block 3 offset 3; seq 1 opens block 1
    assert slots == [15, 4]
    assert bm.block_table(1) == ([9, 0, 1], 9)
    slots, _ = bm.step([0])               # seq 0's last block is full → next free block (2)
    assert slots == [8] and bm.block_table(0) == ([5, 12, 3, 2], 13)


def test_copy_on_write_tie_break():
    bm = OracleBlockManager(8, 4, list(range(8)))
    bm.add_seq(10, 6)                      # blocks 0 (full), 1 (2 tokens)
    bm.fork(10, 11)
    bm.fork(10, 12)
    assert bm.refcount(0) == 3 and bm.refcount(1) == 3
    slots, pairs = bm.step([10, 11, 12])
    # 10 and 11 find block 1 shared and copy it to 2 and 3; 12 finds rc 1 and writes in place
    assert pairs == [(1, 2), (1, 3)]
    assert slots == [2 * 4 + 2, 3 * 4 + 2, 1 * 4 + 2]
    assert bm.block_table(10) == ([0, 2], 7)
    assert bm.block_table(11) == ([0, 3], 7)
    assert bm.block_table(12) == ([0, 1], 7)
    assert [bm.refcount(b) for b in range(4)] == [3, 1, 1, 1]
    assert bm.stats()["cow_copies"] == 2


def test_full_shared_block_needs_no_copy():
    bm = OracleBlockManager(8, 4, list(range(8)))
    bm.add_seq(0, 8)
    bm.fork(0, 1)
    slots, pairs = bm.step([0, 1])
    assert pairs == [] and slots == [8, 12]
    assert bm.refcount(0) == 2 and bm.refcount(1) == 2


def test_pool_exhaustion_leaves_state_unchanged():
    bm = OracleBlockManager(3, 4, [2, 0, 1])
    bm.add_seq(0, 4)
    bm.add_seq(1, 4)
    before = (bm.block_table(0), bm.block_table(1), list(bm.free), list(bm.rc))
    with pytest.raises(NoBlocksError):
        bm.step([0, 1])                   # needs 2 blocks, 1 free
    assert (bm.block_table(0), bm.block_table(1), list(bm.free), list(bm.rc)) == before
    with pytest.raises(NoBlocksError):
        bm.add_seq(2, 5)
    assert 2 not in bm.seqs


def test_exhaustion_counts_in_batch_copies():
    # two sharers of a partial block: the first copies, the second writes in place
    bm = OracleBlockManager(3, 4, [0, 1, 2])
    bm.add_seq(0, 2)
    bm.fork(0, 1)
    bm.add_seq(2, 4)                      # uses block 1; block 2 free
    with pytest.raises(NoBlocksError):
        bm.step([0, 1, 2])                # needs a copy for 0 and a new block for 2
    slots, pairs = bm.step([0, 1])        # exactly one free block suffices
    assert pairs == [(0, 2)] and slots == [2 * 4 + 2, 0 * 4 + 2]


def test_free_returns_blocks_fifo():
    bm = OracleBlockManager(6, 2, [4, 1, 3, 0, 5, 2])
    bm.add_seq(0, 5)                      # 4, 1, 3
    bm.add_seq(1, 2)                      # 0
    bm.fork(1, 2)
    bm.free_seq(0)
    assert list(bm.free) == [5, 2, 4, 1, 3]
    bm.free_seq(1)                        # block 0 still held by seq 2
    assert list(bm.free) == [5, 2, 4, 1, 3]
    bm.free_seq(2)
    assert list(bm.free) == [5, 2, 4, 1, 3, 0]


def test_rejects_bad_calls():
    bm = OracleBlockManager(4, 4)
    bm.add_seq(0, 1)
    with pytest.raises(KeyError):
        bm.add_seq(0, 1)
    with pytest.raises(KeyError):
        bm.fork(9, 1)
    with pytest.raises(ValueError):
        bm.step([0, 0])
    with pytest.raises(KeyError):
        bm.step([3])
    with pytest.raises(ValueError):
        OracleBlockManager(3, 4, [0, 1, 1])


def test_sharing_ratio_and_utilisation():
    bm = OracleBlockManager(64, 4)
    bm.add_seq(0, 16)                     # 4 full blocks
    for c in range(1, 8):
        bm.fork(0, c)
    st_ = bm.stats()
    assert accounting.sharing_ratio(st_) == 8.0
    assert accounting.stats_utilisation(st_) == 1.0
    bm.step(list(range(8)))               # each opens one block holding one token
    st_ = bm.stats()
    assert st_["used_blocks"] == 12 and st_["filled_slots"] == 16 + 8
    assert accounting.stats_utilisation(st_) == 24 / 48


class BMStateMachine(RuleBasedStateMachine):
    """Random add/fork/step/swap/free sequences; invariants hold after every call.
    A swap moves the simulated pool's tags of the returned blocks to a host copy
    and back into the blocks swap-in returns, so the read-back invariant checks
    that a sequence comes back with its own tokens in order."""

    def __init__(self):
        super().__init__()
        self.bs = 4
        self.nb = 24
        self.bm = OracleBlockManager(self.nb, self.bs, list(reversed(range(self.nb))))
        self.next_id = 0
        self.contents = {}   # seq id → list of token tags, in logical order
        self.slot_tag = {}   # flat slot → tag written there (a simulated pool)
        self.host = {}       # swapped seq id → tags of its blocks, in table order

    def _write(self, seq, t, slot):
        tag = (seq, t, self.next_id)
        self.next_id += 1
        self.slot_tag[slot] = tag
        self.contents[seq].append(tag)

    @rule(n=st.integers(0, 9))
    def add(self, n):
        sid = self.next_id
        self.next_id += 1
        try:
            self.bm.add_seq(sid, n)
        except NoBlocksError:
            return
        self.contents[sid] = []
        for t, slot in enumerate(self.bm.token_slots(sid)):
            self._write(sid, t, slot)

    @precondition(lambda self: self.bm.seqs)
    @rule(data=st.data())
    def fork(self, data):
        parent = data.draw(st.sampled_from(sorted(self.bm.seqs)))
        child = self.next_id
        self.next_id += 1
        self.bm.fork(parent, child)
        self.contents[child] = list(self.contents[parent])

    @precondition(lambda self: self.bm.seqs)
    @rule(data=st.data())
    def step(self, data):
        ids = data.draw(st.lists(st.sampled_from(sorted(self.bm.seqs)), min_size=1, unique=True))
        lens = {s: self.bm.length(s) for s in ids}
        try:
            slots, pairs = self.bm.step(ids)
        except NoBlocksError:
            assert all(self.bm.length(s) == lens[s] for s in ids)
            return
        # apply copies (whole blocks), then writes, to the simulated pool
        for src, dst in pairs:
            for off in range(self.bs):
                if src * self.bs + off in self.slot_tag:
                    self.slot_tag[dst * self.bs + off] = self.slot_tag[src * self.bs + off]
        for s, slot in zip(ids, slots):
            assert slot // self.bs == self.bm.block_table(s)[0][lens[s] // self.bs]
            self._write(s, lens[s], slot)

    @precondition(lambda self: self.bm.seqs)
    @rule(data=st.data())
    def swap_out(self, data):
        sid = data.draw(st.sampled_from(sorted(self.bm.seqs)))
        table = self.bm.block_table(sid)[0]
        blocks = self.bm.swap_out(sid)
        assert blocks == table and sid not in self.bm.seqs
        self.host[sid] = [[self.slot_tag.get(b * self.bs + o) for o in range(self.bs)] for b in blocks]

    @precondition(lambda self: self.bm.swapped)
    @rule(data=st.data())
    def swap_in(self, data):
        sid = data.draw(st.sampled_from(sorted(self.bm.swapped)))
        free_before = list(self.bm.free)
        try:
            blocks = self.bm.swap_in(sid)
        except NoBlocksError:
            assert list(self.bm.free) == free_before and sid in self.bm.swapped
            return
        assert blocks == free_before[:len(blocks)]                   # taken from the head of the free list
        assert all(self.bm.refcount(b) == 1 for b in blocks)
        for b, tags in zip(blocks, self.host.pop(sid)):
            for o, tag in enumerate(tags):
                if tag is not None:
                    self.slot_tag[b * self.bs + o] = tag

    @precondition(lambda self: self.bm.seqs or self.bm.swapped)
    @rule(data=st.data())
    def free(self, data):
        sid = data.draw(st.sampled_from(sorted(list(self.bm.seqs) + list(self.bm.swapped))))
        self.bm.free_seq(sid)
        del self.contents[sid]
        self.host.pop(sid, None)

    @invariant()
    def refcounts_match_owners(self):
        owners = [0] * self.nb
        for sid in self.bm.seqs:
            for b in self.bm.block_table(sid)[0]:
                owners[b] += 1
        assert owners == [self.bm.refcount(b) for b in range(self.nb)]

    @invariant()
    def free_and_used_partition_the_pool(self):
        free = list(self.bm.free)
        assert len(set(free)) == len(free)
        used = {b for b in range(self.nb) if self.bm.refcount(b) > 0}
        assert used.isdisjoint(free) and used | set(free) == set(range(self.nb))

    @invariant()
    def swapped_sequences_hold_no_blocks(self):
        assert set(self.bm.swapped).isdisjoint(self.bm.seqs)
        st_ = self.bm.stats()
        assert st_["swapped_seqs"] == len(self.bm.swapped)
        assert st_["swapped_tokens"] == sum(len(self.contents[s]) for s in self.bm.swapped)

    @invariant()
    def tables_cover_lengths(self):
        for sid in self.bm.seqs:
            table, n = self.bm.block_table(sid)
            assert len(table) == -(-n // self.bs)

    @invariant()
    def every_sequence_reads_its_own_tokens(self):
        # the simulated pool seen through each table reproduces what the
        # sequence wrote (copy-on-write kept sharers from clobbering each other)
        for sid in self.bm.seqs:
            seen = [self.slot_tag.get(s) for s in self.bm.token_slots(sid)]
            assert seen == self.contents[sid]

    @invariant()
    def waste_is_last_block_padding(self):
        st_ = self.bm.stats()
        assert 0 <= st_["used_blocks"] * self.bs - st_["filled_slots"]
        private_pad = sum(len(self.bm.block_table(s)[0]) * self.bs - self.bm.length(s) for s in self.bm.seqs)
        assert st_["logical_blocks"] * self.bs - st_["logical_tokens"] == private_pad


TestBMStateMachine = BMStateMachine.TestCase
TestBMStateMachine.settings = settings(max_examples=150, stateful_step_count=40, deadline=None)


def test_dispatch_order_hand_example():
    """Parent P (32 tokens, 2 blocks of 16) forked into C1 and C2, which then
    grow to 37 and 34 tokens; D has 50 tokens of its own; E is empty.  Batch
    [E, C2, D, P, C1]: D's group is longest (50) and goes first, then the P
    group by length (C1 37, C2 34, P 32), then E.  A second batch ties two
    groups at length 32 (F, 32 tokens of its own): the group seen first in the
    batch goes first."""
    bm = OracleBlockManager(32, 16)
    bm.add_seq("P", 32)
    bm.fork("P", "C1")
    bm.fork("P", "C2")
    for _ in range(5):
        bm.append_slot("C1")
    for _ in range(2):
        bm.append_slot("C2")
    bm.add_seq("D", 50)
    bm.add_seq("E", 0)
    assert bm.dispatch_order(["E", "C2", "D", "P", "C1"]) == [2, 4, 1, 3, 0]
    bm.add_seq("F", 32)
    assert bm.dispatch_order(["F", "P", "E"]) == [0, 1, 2]
    assert bm.dispatch_order(["P", "F", "E"]) == [0, 1, 2]
    assert bm.dispatch_order(["E", "F", "C2", "P"]) == [2, 3, 1, 0]


def test_dispatch_order_without_sharing_is_a_stable_length_sort():
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.choice([0, 1, 5, 16, 17, 40], size=60)]
    bm = OracleBlockManager(600, 4)
    for i, n in enumerate(lens):
        bm.add_seq(i, n)
    batch = [int(x) for x in rng.permutation(60)]
    want = sorted(range(60), key=lambda p: -lens[batch[p]])     # Python's sort is stable
    assert bm.dispatch_order(batch) == want


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 40), st.integers(0, 3), st.integers(0, 9)), min_size=1, max_size=24))
def test_dispatch_order_properties(spec):
    """Each spec entry adds a root of n tokens with k forks, each fork grown by
    g tokens.  Any batch order: a permutation; a group (same first block) is
    contiguous; group maxima never rise; lengths never rise inside a group."""
    bm = OracleBlockManager(4096, 4)
    ids = []
    for r, (n, k, g) in enumerate(spec):
        bm.add_seq((r, 0), n)
        ids.append((r, 0))
        for c in range(1, k + 1):
            bm.fork((r, 0), (r, c))
            for _ in range(g * c % 7):
                bm.append_slot((r, c))
            ids.append((r, c))
    order = bm.dispatch_order(ids)
    assert sorted(order) == list(range(len(ids)))
    seq = [ids[p] for p in order]
    first = [bm.block_table(s)[0][0] if bm.block_table(s)[0] else ("empty", s) for s in seq]
    length = [bm.length(s) for s in seq]
    runs = []
    for f, n in zip(first, length):
        if runs and runs[-1][0] == f:
            runs[-1][1].append(n)
        else:
            runs.append((f, [n]))
    assert len({r[0] for r in runs}) == len(runs)                # contiguous groups
    maxima = [max(r[1]) for r in runs]
    assert maxima == sorted(maxima, reverse=True)
    for _, ns in runs:
        assert ns == sorted(ns, reverse=True)


def test_prefix_groups_hand_example():
    """P holds 40 tokens (blocks of 16: two full, one with 8); A and B fork
    from P and A appends 3 tokens, which copies the shared third block.  The
    run P, A, B shares two full blocks (32 tokens); X is alone (0)."""
    bm = OracleBlockManager(64, 16)
    bm.add_seq("P", 40)
    bm.fork("P", "A")
    bm.fork("P", "B")
    for _ in range(3):
        bm.append_slot("A")
    bm.add_seq("X", 20)
    assert bm.prefix_groups(["P", "A", "B", "X"]) == ([0, 3, 4], [32, 32, 32, 0], 3)
    assert bm.prefix_groups(["X", "P", "A", "B"]) == ([0, 1, 4], [0, 32, 32, 32], 3)
    # a sibling placed apart starts a run of its own
    assert bm.prefix_groups(["P", "X", "A"]) == ([0, 1, 2, 3], [0, 0, 0], 1)
    # B alone with P: the third block is shared but holds 8 tokens, so only two count
    assert bm.prefix_groups(["P", "B"]) == ([0, 2], [32, 32], 2)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 70), st.integers(0, 3), st.integers(0, 40)), min_size=1, max_size=12),
       st.randoms(use_true_random=False))
def test_prefix_groups_properties(spec, rnd):
    """Random fork families in a random batch order: runs are maximal and
    contiguous, a prefix is whole blocks that every member holds, full and in
    the same place, and it cannot grow by one more such block."""
    bs = 4
    bm = OracleBlockManager(8192, bs)
    ids = []
    for r, (n, k, g) in enumerate(spec):
        bm.add_seq((r, 0), n)
        ids.append((r, 0))
        for c in range(1, k + 1):
            bm.fork((r, 0), (r, c))
            for _ in range((g * c) % 9):
                bm.append_slot((r, c))
            ids.append((r, c))
    rnd.shuffle(ids)
    starts, prefix, largest = bm.prefix_groups(ids)
    assert starts[0] == 0 and starts[-1] == len(ids) and starts == sorted(set(starts))
    assert largest == max(b - a for a, b in zip(starts, starts[1:]))
    for a, b in zip(starts, starts[1:]):
        members = ids[a:b]
        tables = [bm.block_table(s)[0] for s in members]
        firsts = [t[0] if t else None for t in tables]
        assert all(f is not None and f == firsts[0] for f in firsts) or b - a == 1
        if b < len(ids) and firsts[0] is not None:                       # maximal run
            nxt = bm.block_table(ids[b])[0]
            assert not nxt or nxt[0] != firsts[0]
        p = prefix[a]
        assert all(prefix[i] == p for i in range(a, b)) and p % bs == 0
        if b - a == 1:
            assert p == 0
            continue
        nb = p // bs
        assert all(bm.length(s) >= p for s in members)
        assert all(t[:nb] == tables[0][:nb] for t in tables)
        grow_ok = (all(bm.length(s) >= p + bs for s in members) and
                   all(len(t) > nb and t[nb] == tables[0][nb] for t in tables))
        assert not grow_ok


def test_swap_hand_example(example):
    """The worked example's sequence (10 tokens in blocks 5, 12, 3) swapped out
    and back: the blocks come back in table order and rejoin the free tail;
    swap-in takes the head of the free list.  A forked sharer's swap-out only
    drops refcounts, and it comes back with private blocks."""
    bs = example["block_size"]
    table = example["block_table"]
    order = table + [b for b in range(16) if b not in table]
    bm = OracleBlockManager(16, bs, order)
    bm.add_seq(0, example["num_tokens"])
    head = list(bm.free)[:3]
    assert bm.swap_out(0) == table
    assert list(bm.free)[-3:] == table and bm.stats()["swapped_seqs"] == 1
    assert bm.stats()["swapped_tokens"] == example["num_tokens"]
    with pytest.raises(KeyError):
        bm.block_table(0)
    assert bm.swap_in(0) == head
    assert bm.block_table(0) == (head, example["num_tokens"])
    bm.fork(0, 1)
    assert all(bm.refcount(b) == 2 for b in head)
    assert bm.swap_out(1) == head and all(bm.refcount(b) == 1 for b in head)
    back = bm.swap_in(1)
    assert set(back).isdisjoint(head) and all(bm.refcount(b) == 1 for b in back)
    with pytest.raises(KeyError):
        bm.swap_in(1)                                                 # not swapped out any more
