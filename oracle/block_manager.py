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

  * codebumble.net, "CUDA Shared Memory Optimization" (prefix caching): full blocks of token
    ids form a prefix tree; a new prompt follows the tree from its first block and points its
    block table at every block it finds, so those tokens need no prefill.

Readings taken where the pages are silent (listed in the design notes): sequence ids are
integers; freed blocks go to the tail of the free list, in table order; the reference count of
a block is the number of block tables that list it; a call that cannot get every block it needs
changes nothing.  Prefix tree: a node is keyed by its parent node and its block's token ids
(exact comparison); only full prompt blocks are registered; a released registered block stays
findable while it sits in the free list, and is forgotten when it is handed out again.
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
        self.nodes: dict[tuple, int] = {}        # (parent node, block tokens) -> block
        self.node_id: dict[int, int] = {}        # block -> its node id
        self.node_key: dict[int, tuple] = {}     # block -> its key
        self.node_count = 0

    # -- derived state, recomputed from the tables every time (no incremental bookkeeping)
    def users(self, block: int) -> int:
        return sum(t.count(block) for t in self.tables.values())

    # -- operations
    def _take_free(self) -> int:
        block = self.free.pop(0)
        if block in self.node_id:                # handed out again: forget its prefix node
            del self.nodes[self.node_key.pop(block)]
            del self.node_id[block]
        return block

    def _write_one(self, seq: int):
        """Place the next token of `seq`; returns (slot, copy) where copy is None or (old, new)."""
        table = self.tables.setdefault(seq, [])
        pos = self.lengths.get(seq, 0)
        logical, offset = divmod(pos, self.block_size)
        copy = None
        if offset == 0:
            if not self.free:
                raise OutOfBlocks
            table.append(self._take_free())
        elif self.users(table[logical]) > 1:
            if not self.free:
                raise OutOfBlocks
            fresh = self._take_free()
            copy = (table[logical], fresh)
            table[logical] = fresh
        self.lengths[seq] = pos + 1
        return table[logical] * self.block_size + offset, copy

    def append(self, seq_ids):
        """One token per listed id, in order.  All or nothing."""
        saved = self._snapshot()
        slots, copies = [], []
        try:
            for s in seq_ids:
                slot, copy = self._write_one(int(s))
                slots.append(slot)
                if copy is not None:
                    copies.append(copy)
        except OutOfBlocks:
            self._restore(saved)
            raise
        return slots, copies

    def _snapshot(self):
        return (list(self.free), {k: list(v) for k, v in self.tables.items()}, dict(self.lengths),
                dict(self.nodes), dict(self.node_id), dict(self.node_key), self.node_count)

    def _restore(self, saved):
        (self.free, self.tables, self.lengths, self.nodes, self.node_id, self.node_key,
         self.node_count) = saved

    def append_prompt(self, seq: int, tokens):
        """Start `seq` with a prompt: reuse the registered blocks its leading full blocks match,
        allocate the rest, register the full blocks it fills.  Returns (slots, cached tokens)."""
        if seq in self.tables:
            raise KeyError(seq)
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        saved = self._snapshot()
        table, parent, k = [], -1, 0
        while (k + 1) * bs <= len(tokens):
            key = (parent, tuple(tokens[k * bs:(k + 1) * bs]))
            if key not in self.nodes:
                break
            block = self.nodes[key]
            if block in self.free:                # waiting in the free list: take it back
                self.free.remove(block)
            table.append(block)
            parent = self.node_id[block]
            k += 1
        cached = k * bs
        try:
            while k * bs < len(tokens):
                if not self.free:
                    raise OutOfBlocks
                block = self._take_free()
                table.append(block)
                if (k + 1) * bs <= len(tokens):
                    key = (parent, tuple(tokens[k * bs:(k + 1) * bs]))
                    self.nodes[key] = block
                    self.node_id[block] = self.node_count
                    self.node_key[block] = key
                    parent = self.node_count
                    self.node_count += 1
                k += 1
        except OutOfBlocks:
            self._restore(saved)
            raise
        self.tables[seq] = table
        self.lengths[seq] = len(tokens)
        return [table[p // bs] * bs + p % bs for p in range(len(tokens))], cached

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
