"""Pins of the oracle block allocator and slot map (brute-force invariants)."""
import numpy as np
import pytest

from oracle import kvcache as okv


def _check_tables(alloc, lens, num_blocks):
    tabs = alloc.table_rows()
    used = []
    for s, n in enumerate(lens):
        row = tabs[s]
        k = -(-n // 16)
        assert all(b >= 0 for b in row[:k]) and all(b == -1 for b in row[k:])
        used += row[:k]
    assert len(used) == len(set(used))                       # disjoint
    assert set(used) <= set(range(num_blocks))               # within the pool
    assert len(used) + len(alloc.free) == num_blocks         # nothing lost


def test_alloc_takes_free_list_head_in_order():
    order = [5, 3, 0, 7, 1, 2, 6, 4]
    a = okv.BlockAllocator(8, order, 3, 4)
    a.alloc(0, 17)      # 2 blocks
    a.alloc(1, 16)      # 1 block
    a.alloc(2, 1)       # 1 block
    assert a.table_rows() == [[5, 3, -1, -1], [0, -1, -1, -1], [7, -1, -1, -1]]
    a.alloc(0, 33)      # grows by one: next head
    assert a.table_rows()[0] == [5, 3, 1, -1]
    a.alloc(0, 20)      # already big enough: no change
    assert a.table_rows()[0] == [5, 3, 1, -1]


def test_free_returns_blocks_to_tail_in_table_order():
    a = okv.BlockAllocator(6, [0, 1, 2, 3, 4, 5], 2, 4)
    a.alloc(0, 40)      # 0 1 2
    a.alloc(1, 10)      # 3
    a.free_seq(0)
    assert list(a.free) == [4, 5, 0, 1, 2]
    a.alloc(1, 48)      # grows by 2 from the head: 4 5
    assert a.table_rows()[1] == [3, 4, 5, -1]


def test_exhaustion_is_all_or_nothing():
    a = okv.BlockAllocator(4, [3, 2, 1, 0], 2, 8)
    a.alloc(0, 32)
    before = (a.table_rows(), list(a.free))
    with pytest.raises(okv.NoBlocks):
        a.alloc(1, 3 * 16 + 1)
    assert (a.table_rows(), list(a.free)) == before
    with pytest.raises(okv.BadShape):
        a.alloc(0, 9 * 16)
    assert (a.table_rows(), list(a.free)) == before


def test_random_tables_are_disjoint_and_sized():
    rng = np.random.default_rng(0)
    for trial in range(20):
        lens = rng.integers(1, 200, size=rng.integers(1, 12)).tolist()
        need = sum(-(-n // 16) for n in lens)
        nb = need + int(rng.integers(0, 5))
        a = okv.BlockAllocator(nb, rng.permutation(nb), len(lens), 13)
        for s, n in enumerate(lens):
            a.alloc(s, n)
        _check_tables(a, lens, nb)


def test_slot_map_equals_flat_expansion_of_the_table():
    rng = np.random.default_rng(1)
    lens = [1, 15, 16, 17, 100]
    nb = 20
    a = okv.BlockAllocator(nb, rng.permutation(nb), len(lens), 8)
    for s, n in enumerate(lens):
        a.alloc(s, n)
    tabs = a.table_rows()
    row_seq, row_pos, expect = [], [], []
    for s, n in enumerate(lens):
        flat = [b * 16 + i for b in tabs[s] if b >= 0 for i in range(16)]
        for p in range(n):
            row_seq.append(s)
            row_pos.append(p)
            expect.append(flat[p])
    row_seq.append(-1)
    row_pos.append(3)
    expect.append(-1)
    assert okv.slot_map(tabs, row_seq, row_pos) == expect
    slots = [x for x in expect if x >= 0]
    assert len(slots) == len(set(slots))   # no two positions share a slot
