"""Host block manager: allocation on fill, forking by reference, copy-on-write
of a shared partly filled block, release at reference count zero, pool
exhaustion."""

import numpy as np
import pytest

from workloads import BlockPool, PoolExhausted


def test_allocates_only_when_block_full():
    pool = BlockPool(10, 4)
    s = pool.new_sequence()
    allocs = []
    for t in range(9):
        before = pool.num_free
        slot, cow = pool.append_slot(s)
        assert cow is None
        allocs.append(before - pool.num_free)
        assert slot == s.block_table[t // 4] * 4 + t % 4
    assert allocs == [1, 0, 0, 0, 1, 0, 0, 0, 1]
    assert len(s.block_table) == 3 == -(-9 // 4)


def test_free_order_follows_given_permutation():
    order = list(np.random.default_rng(0).permutation(6))
    pool = BlockPool(6, 2, order=order)
    s = pool.new_sequence()
    for _ in range(6):
        pool.append_slot(s)
    assert s.block_table == order[:3]


def test_fork_shares_by_reference():
    pool = BlockPool(8, 4)
    a = pool.new_sequence()
    for _ in range(5):
        pool.append_slot(a)
    b = pool.fork(a)
    c = pool.fork(a)
    assert b.block_table == a.block_table == c.block_table
    assert [pool.ref[x] for x in a.block_table] == [3, 3]
    assert pool.num_free == 6
    assert pool.shared_ratio() == 1.0


def test_cow_on_shared_partial_block():
    pool = BlockPool(16, 4)
    parent = pool.new_sequence()
    for _ in range(6):                       # last block holds 2 of 4
        pool.append_slot(parent)
    sharers = [parent] + [pool.fork(parent) for _ in range(3)]
    last = parent.block_table[-1]
    pairs = []
    for s in sharers:
        _, cow = pool.append_slot(s)
        if cow:
            pairs.append(cow)
    # every holder but the last copies; the last writes in place
    assert len(pairs) == 3
    assert all(src == last for src, _ in pairs)
    assert len({dst for _, dst in pairs}) == 3
    assert sharers[-1].block_table[-1] == last
    assert pool.ref[last] == 1
    assert pool.ref[parent.block_table[0]] == 4          # full prompt block still shared


def test_no_cow_when_shared_block_is_full():
    pool = BlockPool(8, 4)
    a = pool.new_sequence()
    for _ in range(4):
        pool.append_slot(a)
    b = pool.fork(a)
    _, cow = pool.append_slot(b)
    assert cow is None and len(b.block_table) == 2 and pool.ref[a.block_table[0]] == 2


def test_free_returns_blocks_at_zero():
    pool = BlockPool(4, 2)
    a = pool.new_sequence()
    for _ in range(4):
        pool.append_slot(a)
    b = pool.fork(a)
    pool.free(a)
    assert pool.num_free == 2            # still referenced by b
    pool.free(b)
    assert pool.num_free == 4 and pool.blocks_in_use() == 0


def test_pool_exhaustion_raises():
    pool = BlockPool(2, 2)
    s = pool.new_sequence()
    for _ in range(4):
        pool.append_slot(s)
    with pytest.raises(PoolExhausted):
        pool.append_slot(s)


def test_bad_order_rejected():
    with pytest.raises(AssertionError):
        BlockPool(3, 2, order=[0, 0, 1])
