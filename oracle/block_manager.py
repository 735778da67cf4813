"""Reference model of the block manager (test infrastructure, plain Python).

Written from the pages' description, not from the library:
  * codebumble.net, "The Block Table Mapping Subsystem": the cache is split into physical
    blocks; a token at position p belongs to logical block p // block_size at offset
    p % block_size; a physical block is taken from a global free list (its head) when a token
    opens a new logical block, and appended to the sequence's block table.  The section
    "Continuous Batching" returns a finished sequence's blocks to the free list.
  * bicarait.com, "Architectural Blueprint 2", and infoisland, section 2: branches of one
    prompt point at the same physical blocks; a block is duplicated only when a branch writes
    into a block that other branches still use (copy-on-write).

Readings taken where the pages are silent (listed in the design notes): sequence ids are
integers; freed blocks go to the tail of the free list, in table order; the reference count of
a block is the number of block tables that list it; a call that cannot get every block it needs
changes nothing.
"""

from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.free = list(range(num_blocks))
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}

    # -- derived state, recomputed from the tables every time (no incremental bookkeeping)
    def users(self, block: int) -> int:
        return sum(t.count(block) for t in self.tables.values())

    # -- operations
    def _write_one(self, seq: int):
        """Place the next token of `seq`; returns (slot, copy) where copy is None or (old, new)."""
        table = self.tables.setdefault(seq, [])
        pos = self.lengths.get(seq, 0)
        logical, offset = divmod(pos, self.block_size)
        copy = None
        if offset == 0:
            if not self.free:
                raise OutOfBlocks
            table.append(self.free.pop(0))
        elif self.users(table[logical]) > 1:
            if not self.free:
                raise OutOfBlocks
            fresh = self.free.pop(0)
            copy = (table[logical], fresh)
            table[logical] = fresh
        self.lengths[seq] = pos + 1
        return table[logical] * self.block_size + offset, copy

    def append(self, seq_ids):
        """One token per listed id, in order.  All or nothing."""
        saved = (list(self.free), {k: list(v) for k, v in self.tables.items()}, dict(self.lengths))
        slots, copies = [], []
        try:
            for s in seq_ids:
                slot, copy = self._write_one(int(s))
                slots.append(slot)
                if copy is not None:
                    copies.append(copy)
        except OutOfBlocks:
            self.free, self.tables, self.lengths = saved
            raise
        return slots, copies

    def fork(self, parent: int, child: int):
        if parent not in self.tables or child in self.tables:
            raise KeyError((parent, child))
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]

    def release(self, seq: int):
        table = self.tables.pop(seq)
        del self.lengths[seq]
        for b in table:
            if self.users(b) == 0:
                self.free.append(b)

    def block_table(self, seq: int, width: int):
        t = self.tables[seq]
        return t + [-1] * (width - len(t)), self.lengths[seq]
