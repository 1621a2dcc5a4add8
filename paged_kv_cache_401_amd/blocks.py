"""Host-side block manager: free list, per-sequence block tables, reference
counts and copy-on-write decisions for a pool of fixed-size KV blocks.

It produces the three index inputs of the device entry points: block tables,
slot mappings and (src, dst) copy pairs.  It runs on the host and touches no
KV data.

Rules followed (source pages by title and section):
- "PagedAttention" glossary page (Ultralytics), how paging works: a sequence
  takes a new block only when its last one is full, from any free location;
  the table records the order; the worked example pops free blocks from the
  front of a free list, and token ``pos`` goes to slot ``pos % 16`` of block
  ``table[pos // 16]``.
- Same page, sharing blocks between sequences: tables of several sequences
  may name one physical block, with a per-block reference count; a sequence
  about to write into a block that others still use copies it first.
- Russian page on PagedAttention in vLLM, "two answers to one request": full
  shared blocks stay shared; only the block that has to split is copied;
  blocks left without references are freed.
- Same page, logical order vs physical placement: the prompt is allocated
  first, then the last block fills, and a new block is added only when needed.
  (The French dev.to article says every new token takes a block from the free
  list; the two other pages are followed.)
"""
from __future__ import annotations

from dataclasses import dataclass, field

BLOCK_SIZE = 16


class NoFreeBlock(RuntimeError):
    """The pool has no free block left."""


@dataclass
class _Seq:
    table: list = field(default_factory=list)
    length: int = 0
    on_host: bool = False   # table lists host slots while swapped out


class BlockManager:
    def __init__(self, num_blocks: int, free_list=None, block_size: int = BLOCK_SIZE,
                 num_host_slots: int = 0):
        if block_size != BLOCK_SIZE:
            raise ValueError("block size is fixed at 16 tokens")
        self.num_blocks = int(num_blocks)
        self.block_size = block_size
        self.free = list(range(num_blocks)) if free_list is None else [int(b) for b in free_list]
        if len(set(self.free)) != len(self.free) or any(
                b < 0 or b >= num_blocks for b in self.free):
            raise ValueError("free list must hold distinct block ids inside the pool")
        self.refcount = [0] * self.num_blocks
        self.seqs: dict = {}
        # host slots for swapped-out blocks, with their reference counts
        self.num_host_slots = int(num_host_slots)
        self.host_free = list(range(self.num_host_slots))
        self.host_refcount = [0] * self.num_host_slots
        # event counters (allocations, copies, frees) for accounting reports
        self.n_alloc = 0
        self.n_cow = 0
        self.n_freed = 0

    # ----------------------------------------------------------- allocation
    def _allocate(self) -> int:
        if not self.free:
            raise NoFreeBlock("no free block in a pool of %d" % self.num_blocks)
        b = self.free.pop(0)
        self.refcount[b] = 1
        self.n_alloc += 1
        return b

    def add_sequence(self, seq_id) -> None:
        if seq_id in self.seqs:
            raise KeyError("sequence %r exists" % (seq_id,))
        self.seqs[seq_id] = _Seq()

    def append_tokens(self, seq_id, n: int):
        """Reserve slots for ``n`` new tokens of ``seq_id``.

        Returns ``(slots, cow_pairs)``: the slot of each new token, and the
        (src, dst) block copies that must run before those tokens are written.
        """
        seq = self.seqs[seq_id]
        if seq.on_host:
            raise RuntimeError("sequence %r is swapped out" % (seq_id,))
        n = int(n)
        if n < 0:
            raise ValueError("cannot append %d tokens" % n)
        # all or nothing: the blocks this call takes -- one per block boundary
        # crossed, plus a copy of a shared, partly filled last block -- must
        # all be free before anything changes
        bs = self.block_size
        need = -(-(seq.length + n) // bs) - -(-seq.length // bs)
        if n > 0 and seq.length % bs != 0 and self.refcount[seq.table[-1]] > 1:
            need += 1
        if need > len(self.free):
            raise NoFreeBlock("%d tokens need %d free blocks, %d left" % (n, need, len(self.free)))
        slots, pairs = [], []
        for _ in range(n):
            pos = seq.length
            if pos % self.block_size == 0:
                seq.table.append(self._allocate())
            else:
                last = seq.table[-1]
                if self.refcount[last] > 1:
                    new = self._allocate()
                    pairs.append((last, new))
                    self.refcount[last] -= 1
                    seq.table[-1] = new
                    self.n_cow += 1
            slots.append(seq.table[pos // self.block_size] * self.block_size
                         + pos % self.block_size)
            seq.length += 1
        return slots, pairs

    def fork(self, parent, child) -> None:
        """``child`` starts as a copy of ``parent``'s table, sharing every block."""
        p = self.seqs[parent]
        if p.on_host:
            raise RuntimeError("sequence %r is swapped out" % (parent,))
        self.add_sequence(child)
        c = self.seqs[child]
        c.table = list(p.table)
        c.length = p.length
        for b in p.table:
            self.refcount[b] += 1

    def free_sequence(self, seq_id) -> None:
        seq = self.seqs.pop(seq_id)
        if seq.on_host:
            for h in seq.table:
                self.host_refcount[h] -= 1
                if self.host_refcount[h] == 0:
                    self.host_free.append(h)
            return
        for b in seq.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
                self.n_freed += 1

    # ------------------------------------------------------------- swapping
    def swap_out(self, seq_ids):
        """Move every block of the sequences ``seq_ids`` to host slots, block by
        block (the French page: small pages move to the CPU instead of whole
        sequences).  The group must hold every reference to its blocks, so
        shared blocks move once and stay shared.  Returns the
        (device block, host slot) pairs to copy before the freed blocks are
        reused."""
        group = [self.seqs[s] for s in seq_ids]
        if any(sq.on_host for sq in group):
            raise RuntimeError("a sequence of the group is already swapped out")
        refs, order = {}, []
        for sq in group:
            for b in sq.table:
                if b not in refs:
                    order.append(b)
                refs[b] = refs.get(b, 0) + 1
        if any(self.refcount[b] != refs[b] for b in order):
            raise RuntimeError("a block of the group is shared with a sequence outside it")
        if len(order) > len(self.host_free):
            raise NoFreeBlock("no free host slot for %d blocks" % len(order))
        slot_of = {b: self.host_free.pop(0) for b in order}
        for b in order:
            h = slot_of[b]
            self.host_refcount[h] = self.refcount[b]
            self.refcount[b] = 0
            self.free.append(b)
        for sq in group:
            sq.table = [slot_of[b] for b in sq.table]
            sq.on_host = True
        return [(b, slot_of[b]) for b in order]

    def swap_in(self, seq_ids):
        """Bring the swapped-out sequences ``seq_ids`` back into free device
        blocks (any free location, as for new blocks).  Returns the
        (device block, host slot) pairs to copy before they are attended."""
        group = [self.seqs[s] for s in seq_ids]
        if not all(sq.on_host for sq in group):
            raise RuntimeError("a sequence of the group is not swapped out")
        order = []
        for sq in group:
            for h in sq.table:
                if h not in order:
                    order.append(h)
        if len(order) > len(self.free):
            raise NoFreeBlock("no free device block for %d slots" % len(order))
        block_of = {}
        for h in order:
            b = self.free.pop(0)
            block_of[h] = b
            self.refcount[b] = self.host_refcount[h]
            self.host_refcount[h] = 0
            self.host_free.append(h)
        for sq in group:
            sq.table = [block_of[h] for h in sq.table]
            sq.on_host = False
        return [(block_of[h], h) for h in order]

    # -------------------------------------------------------------- queries
    def block_table(self, seq_id) -> list:
        return list(self.seqs[seq_id].table)

    def length(self, seq_id) -> int:
        return self.seqs[seq_id].length

    def physical_blocks_in_use(self) -> int:
        return sum(1 for r in self.refcount if r > 0)

    def host_slots_in_use(self) -> int:
        return sum(1 for r in self.host_refcount if r > 0)

    def logical_blocks(self) -> int:
        return sum(len(s.table) for s in self.seqs.values())


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks a sequence of n tokens occupies: ceil(n / block_size)."""
    return -(-int(n_tokens) // block_size)


def unused_slots(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Slots reserved but unused: only the unfilled part of the last block."""
    return blocks_for(n_tokens, block_size) * block_size - int(n_tokens)


def prefix_groups(tables, context_lens, sizes, max_group: int):
    """Inputs of the prefix-shared decode for a batch cut into groups of
    consecutive sequences: ``sizes`` lists each group's member count in batch
    order, and a group's shared prefix is the number of leading whole blocks
    (full in every member's context) that every member's table names alike --
    the blocks a fork left shared ("PagedAttention" glossary page, sharing
    blocks between sequences).  Groups larger than ``max_group`` are cut.
    Returns (group_start [G + 1], prefix_blocks [G]) as int lists."""
    starts, prefix = [0], []
    s = 0
    for size in sizes:
        size = int(size)
        while size > 0:
            m = min(size, max_group)
            members = range(s, s + m)
            whole = min(int(context_lens[t]) // BLOCK_SIZE for t in members)
            k = 0
            while k < whole and all(int(tables[t][k]) == int(tables[s][k]) for t in members):
                k += 1
            prefix.append(k)
            s += m
            starts.append(s)
            size -= m
    if s != len(context_lens):
        raise ValueError("group sizes cover %d of %d sequences" % (s, len(context_lens)))
    return starts, prefix
