"""Oracle: paged KV-cache block allocator and token -> slot mapping.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "gpu-waiting-not-working" (nanoserve notes), section "What I
changed because of it": the cache is paged -- each sequence owns a list of
fixed-size blocks (its block table) and every token is mapped to a cache slot
through that table.  The pages fix neither an allocation policy nor the slot
arithmetic; the readings taken here are:

* blocks hold 16 slots; the pool's free list starts in a caller-given order
  (identity, or a seeded permutation for fragmented tables);
* ``alloc(seq, n)`` grows ``seq`` to hold ``n`` tokens, taking the missing
  blocks from the head of the free list, all or nothing;
* ``free_seq`` returns the sequence's blocks to the tail, in table order;
* slot = table[seq][pos // 16] * 16 + pos % 16; a padding row (seq < 0) maps
  to -1.
"""
from __future__ import annotations

from collections import deque

BLOCK = 16


class NoBlocks(Exception):
    pass


class BadShape(Exception):
    pass


class BlockAllocator:
    def __init__(self, num_blocks, free_order, max_seqs, max_blocks_per_seq, block_size=BLOCK):
        order = [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free order must be a permutation"
        self.block_size = block_size
        self.free = deque(order)
        self.max_seqs = max_seqs
        self.max_blocks = max_blocks_per_seq
        self.tables = [[] for _ in range(max_seqs)]

    def alloc(self, seq, n_tokens):
        """Grow ``seq`` to hold ``n_tokens`` tokens; all or nothing."""
        if not 0 <= seq < self.max_seqs or n_tokens < 0:
            raise ValueError("bad sequence or token count")
        want = -(-n_tokens // self.block_size)
        if want > self.max_blocks:
            raise BadShape("sequence would exceed its block-table row")
        extra = want - len(self.tables[seq])
        if extra <= 0:
            return
        if extra > len(self.free):
            raise NoBlocks("pool exhausted")
        for _ in range(extra):
            self.tables[seq].append(self.free.popleft())

    def free_seq(self, seq):
        if not 0 <= seq < self.max_seqs:
            raise ValueError("bad sequence")
        self.free.extend(self.tables[seq])
        self.tables[seq] = []

    def table_rows(self):
        """[max_seqs][max_blocks_per_seq] nested list, -1 padded."""
        return [t + [-1] * (self.max_blocks - len(t)) for t in self.tables]


def slot_of(table_row, pos, block_size=BLOCK):
    """Cache slot holding position ``pos`` of a sequence with this table row."""
    return table_row[pos // block_size] * block_size + pos % block_size


def slot_map(tables, row_seq, row_pos, block_size=BLOCK):
    out = []
    for s, p in zip(row_seq, row_pos):
        s, p = int(s), int(p)
        out.append(-1 if s < 0 else slot_of(tables[s], p, block_size))
    return out
