"""Reference block manager (oracle, test-only).

A plain Python statement of the paged KV cache's bookkeeping, written to be
checked by eye against the pages:

* The cache is a pool of fixed-size physical blocks of ``block_size`` token
  slots; a sequence's blocks need not be adjacent ([P1 "Paged Attention 的工作
  原理"], [P2 §2.1]).
* Each sequence owns a block table mapping logical block j to a physical block
  ([P1 "块表（Block Table）"], [P2 §2.3]); token t lives in logical block
  ⌊t / block_size⌋ at offset t mod block_size ([P2 §5], the
  (block index, in-block offset) address).  Its flat slot number is
  ``physical_block * block_size + offset``.
* Prefill of an n-token prompt takes ⌈n / block_size⌉ blocks; the last may be
  part-filled, its tail left as padding ([P2 §3.2.1]).
* Each decode step first checks whether the last block is full; if so a fresh
  block is requested and appended to the table, then the new token's K/V is
  written into its slot ([P2 §3.2.2], steps 2–3; [P1] worked example, steps 1–3).
* Free blocks sit in one list; a finished request returns its blocks there and
  any free block may serve any request ([P2 §3.3]).
* Blocks may be shared between requests by reference count; a shared block is
  read-only, and a write into one first copies it, points the writer's table at
  the copy and drops the old block's count by one ([P2 §3.4]; [P1
  "跨请求的内存共享"]; [P3 "技术洞察"]).  Forked samples and beam branches
  share their parent's blocks this way.

Readings where the pages leave a step open (fixed so that two independent
implementations agree bit for bit):

1. The free list is FIFO, seeded by ``initial_free_order`` (default 0..n-1);
   allocation pops from the head, release appends to the tail.  Any policy is
   valid by [P2 §3.3]; this one is chosen to be reproducible.
2. A batch step visits sequences in batch order.  A sequence copies its last
   block iff that block's refcount is > 1 at its turn, so the last of k sharers
   writes in place (k - 1 copies).  A full-but-shared last block needs no copy:
   the append opens a new block.
3. "Read-only" means refcount > 1.
4. A batch step is all-or-nothing: if the pool cannot supply every block the
   batch needs, nothing changes and ``NoBlocksError`` is raised.
5. ``free_seq`` decrements refcounts in table order; blocks reaching zero join
   the tail of the free list in that order.

Swapping ([P2 §5], [P2 §8]: inactive blocks go to CPU memory and come back,
as pages are swapped): ``swap_out`` hands back a sequence's table (the blocks
whose bytes go to the host) and releases those blocks as ``free_seq`` would;
the sequence keeps only its length.  ``swap_in`` takes ⌈length/bs⌉ fresh
blocks, all private, as its new table (the destinations of the copy back).
Readings: blocks shared before swap-out are not shared again after swap-in;
a swapped sequence is unknown to every other call except ``free_seq``.

``dispatch_order`` is not from the pages: it is the library's scheduling
choice for a decode batch (longest processing time first over groups of
sequences that share their first physical block), stated here so that the
host implementation can be checked against a plain sort.
"""
from collections import deque


class NoBlocksError(RuntimeError):
    """The free list cannot supply the blocks a call needs (state unchanged)."""


class _Seq:
    __slots__ = ("table", "length")

    def __init__(self, table, length):
        self.table = table
        self.length = length


class OracleBlockManager:
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.rc = [0] * num_blocks
        self.seqs = {}
        self.swapped = {}   # seq id -> length while swapped out
        self.cow_copies = 0

    # -- allocation primitives -------------------------------------------------
    def _pop_free(self):
        b = self.free.popleft()
        assert self.rc[b] == 0
        self.rc[b] = 1
        return b

    def _blocks_for(self, n_tokens):
        return -(-n_tokens // self.block_size)

    # -- sequence lifecycle ----------------------------------------------------
    def add_seq(self, seq_id, num_tokens):
        """Prefill allocation: ⌈n/bs⌉ fresh blocks, each with refcount 1."""
        if seq_id in self.seqs or seq_id in self.swapped:
            raise KeyError(f"sequence {seq_id} already exists")
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        need = self._blocks_for(num_tokens)
        if need > len(self.free):
            raise NoBlocksError(f"need {need} blocks, {len(self.free)} free")
        table = [self._pop_free() for _ in range(need)]
        self.seqs[seq_id] = _Seq(table, num_tokens)

    def fork(self, parent_id, child_id):
        """The child shares every block of the parent; each refcount rises by one."""
        if parent_id not in self.seqs:
            raise KeyError(f"unknown parent {parent_id}")
        if child_id in self.seqs or child_id in self.swapped:
            raise KeyError(f"sequence {child_id} already exists")
        parent = self.seqs[parent_id]
        for b in parent.table:
            self.rc[b] += 1
        self.seqs[child_id] = _Seq(list(parent.table), parent.length)

    def _append_needs_block(self, seq, rc_view):
        t = seq.length
        if t % self.block_size == 0:
            return True
        return rc_view(seq.table[-1]) > 1

    def append_slot(self, seq_id):
        """One decode-step append.  Returns (slot, cow_src, cow_dst); -1 = no copy."""
        seq = self.seqs[seq_id]
        t = seq.length
        bs = self.block_size
        cow_src = cow_dst = -1
        if t % bs == 0:
            if not self.free:
                raise NoBlocksError("free list empty")
            seq.table.append(self._pop_free())
        elif self.rc[seq.table[-1]] > 1:
            if not self.free:
                raise NoBlocksError("free list empty")
            old = seq.table[-1]
            new = self._pop_free()
            self.rc[old] -= 1
            seq.table[-1] = new
            cow_src, cow_dst = old, new
            self.cow_copies += 1
        slot = seq.table[t // bs] * bs + t % bs
        seq.length = t + 1
        return slot, cow_src, cow_dst

    def step(self, seq_ids):
        """Batched decode-step append in batch order (all-or-nothing).

        Returns (slots, cow_pairs) where cow_pairs lists (src, dst) in the order
        the copies were decided.
        """
        seq_ids = list(seq_ids)
        if len(set(seq_ids)) != len(seq_ids):
            raise ValueError("a sequence may appear at most once per step")
        for s in seq_ids:
            if s not in self.seqs:
                raise KeyError(f"unknown sequence {s}")
        # Dry run: count the blocks this batch takes, tracking the refcount drops
        # that earlier copies in the same batch cause.
        drops = {}
        need = 0
        for s in seq_ids:
            seq = self.seqs[s]
            if seq.length % self.block_size == 0:
                need += 1
            else:
                last = seq.table[-1]
                if self.rc[last] - drops.get(last, 0) > 1:
                    need += 1
                    drops[last] = drops.get(last, 0) + 1
        if need > len(self.free):
            raise NoBlocksError(f"step needs {need} blocks, {len(self.free)} free")
        slots, pairs = [], []
        for s in seq_ids:
            slot, src, dst = self.append_slot(s)
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        return slots, pairs

    def swap_out(self, seq_id):
        """The sequence's blocks in table order; they are released as by free_seq
        and the sequence keeps only its length."""
        seq = self.seqs[seq_id]
        blocks = list(seq.table)
        self.free_seq(seq_id)
        self.swapped[seq_id] = seq.length
        return blocks

    def swap_in(self, seq_id):
        """⌈length/bs⌉ fresh private blocks as the sequence's new table."""
        length = self.swapped[seq_id]
        need = self._blocks_for(length)
        if need > len(self.free):
            raise NoBlocksError(f"swap-in needs {need} blocks, {len(self.free)} free")
        del self.swapped[seq_id]
        self.seqs[seq_id] = _Seq([self._pop_free() for _ in range(need)], length)
        return list(self.seqs[seq_id].table)

    def free_seq(self, seq_id):
        """Release: refcount -1 per block in table order; zeros rejoin the free tail."""
        if seq_id in self.swapped:
            del self.swapped[seq_id]
            return
        seq = self.seqs.pop(seq_id)
        for b in seq.table:
            self.rc[b] -= 1
            assert self.rc[b] >= 0
            if self.rc[b] == 0:
                self.free.append(b)

    # -- queries ---------------------------------------------------------------
    def block_table(self, seq_id):
        seq = self.seqs[seq_id]
        return list(seq.table), seq.length

    def length(self, seq_id):
        return self.seqs[seq_id].length

    def refcount(self, block):
        return self.rc[block]

    def token_slots(self, seq_id, first=0, count=None):
        """Flat slot numbers of tokens [first, first+count) of a sequence."""
        seq = self.seqs[seq_id]
        if count is None:
            count = seq.length - first
        if first < 0 or count < 0 or first + count > seq.length:
            raise ValueError("token range outside the sequence")
        bs = self.block_size
        return [seq.table[t // bs] * bs + t % bs for t in range(first, first + count)]

    def dispatch_order(self, seq_ids):
        """Batch positions in dispatch order.  A group is the set of batch
        sequences whose first block is the same physical block (an empty
        sequence is alone); groups go longest member first, then by their
        lowest position; inside a group, longer sequences first, then lower
        position."""
        members = {}
        for pos, s in enumerate(seq_ids):
            table = self.seqs[s].table
            group = table[0] if table else ("empty", pos)
            members.setdefault(group, []).append(pos)
        keys = []
        for group, positions in members.items():
            longest = max(self.seqs[seq_ids[p]].length for p in positions)
            for p in positions:
                keys.append((-longest, min(positions), -self.seqs[seq_ids[p]].length, p))
        return [k[3] for k in sorted(keys)]

    def prefix_groups(self, seq_ids):
        """Runs of consecutive batch positions whose first block is the same
        physical block, and for each member the number of leading tokens held
        in blocks that every member of its run shares and that are full in
        every member (0 for a run of one).  Returns (starts + [n], prefix
        tokens per position, largest run)."""
        n = len(seq_ids)
        seqs = [self.seqs[s] for s in seq_ids]
        starts, prefix, largest = [], [0] * n, 0
        a = 0
        while a < n:
            b = a + 1
            if seqs[a].table:
                while b < n and seqs[b].table and seqs[b].table[0] == seqs[a].table[0]:
                    b += 1
            blocks = 0
            if b - a > 1:
                limit = min(seq.length // self.block_size for seq in seqs[a:b])
                while (blocks < limit and
                       all(blocks < len(seq.table) and seq.table[blocks] == seqs[a].table[blocks] for seq in seqs[a:b])):
                    blocks += 1
            starts.append(a)
            for i in range(a, b):
                prefix[i] = blocks * self.block_size
            largest = max(largest, b - a)
            a = b
        return starts + [n], prefix, largest

    def padded_tables(self, seq_ids, stride, pad=-1):
        """Block tables of ``seq_ids`` as rows of ``stride`` entries, padded with ``pad``."""
        rows = []
        for s in seq_ids:
            table = self.seqs[s].table
            if len(table) > stride:
                raise ValueError("stride shorter than a block table")
            rows.append(list(table) + [pad] * (stride - len(table)))
        return rows

    def stats(self):
        """Occupancy counters: see ``oracle.accounting`` for the derived ratios."""
        bs = self.block_size
        fill = {}
        for seq in self.seqs.values():
            for j, b in enumerate(seq.table):
                n = min(bs, seq.length - j * bs)
                # sharers of one block always agree on its fill (a divergent
                # write copies first), so max() only guards the invariant
                fill[b] = max(fill.get(b, 0), n)
        used = [b for b in range(self.num_blocks) if self.rc[b] > 0]
        return {
            "num_blocks": self.num_blocks,
            "block_size": bs,
            "free_blocks": len(self.free),
            "used_blocks": len(used),
            "shared_blocks": sum(1 for b in used if self.rc[b] > 1),
            "num_seqs": len(self.seqs),
            "logical_tokens": sum(s.length for s in self.seqs.values()),
            "logical_blocks": sum(len(s.table) for s in self.seqs.values()),
            "filled_slots": sum(fill.values()),
            "cow_copies": self.cow_copies,
            "swapped_seqs": len(self.swapped),
            "swapped_tokens": sum(self.swapped.values()),
        }
