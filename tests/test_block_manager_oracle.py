"""Pins of the reference BlockManager (CPU): the pages' printed traces."""

import numpy as np
import pytest

import block_trace as T
from oracle.block_manager import BlockManager, Seq, chained_hash


def test_trace_of_seven_rounds():
    T.replay_trace(BlockManager)


def test_prefix_hit_revives_shared_block():
    T.check_prefix_hit(BlockManager)


def test_shared_blocks_diagram():
    T.check_shared_blocks(BlockManager)


def test_chain_depends_on_whole_prefix():
    """Same block contents after different prefixes hash differently; same
    prefix and contents hash the same."""
    rng = np.random.default_rng(3)
    blk = rng.integers(0, 1000, 256).tolist()
    p1, p2 = chained_hash(rng.integers(0, 1000, 256), None), chained_hash(
        rng.integers(0, 1000, 256), None)
    assert chained_hash(blk, p1) != chained_hash(blk, p2)
    assert chained_hash(blk, p1) == chained_hash(list(blk), p1)
    assert chained_hash(blk, None) != chained_hash(blk, 0)


def test_revived_block_after_free_and_stale_entry_dropped():
    """A freed block keeps its hash (a new request revives it); once handed
    out again its old index entry is gone."""
    bm = BlockManager(2, 4)
    a = Seq([1, 2, 3, 4, 5], 4)
    bm.allocate(a, bm.can_allocate(a))
    bm.hash_blocks(a, 5)
    a.num_cached_tokens = 5
    h0 = chained_hash([1, 2, 3, 4], None)
    assert bm.state()["index"] == {h0: 0}
    bm.deallocate(a)  # releases in reverse table order: 1, then 0
    assert bm.state()["free"] == [1, 0] and bm.state()["index"] == {h0: 0}
    b = Seq([1, 2, 3, 4, 9], 4)
    assert bm.can_allocate(b) == 1
    bm.allocate(b, 1)
    assert b.block_table == [0, 1] and bm.state()["ref_count"] == [1, 1]
    bm.deallocate(b)
    c = Seq([7, 7, 7, 7, 7, 7], 4)
    bm.allocate(c, bm.can_allocate(c))  # hands block 0 out again: its entry is dropped
    assert c.block_table == [1, 0] and bm.state()["index"] == {}


@pytest.mark.parametrize("n", [256, 257])
def test_new_block_exactly_after_a_full_one(n):
    bm = BlockManager(3, 256)
    s = Seq(list(range(n)), 256)
    bm.allocate(s, bm.can_allocate(s))
    assert len(s.block_table) == (1 if n == 256 else 2)
    s.token_ids.append(0)
    assert bm.can_append(s)
    before = len(s.block_table)
    bm.may_append(s)
    assert len(s.block_table) == before + (1 if (n + 1) % 256 == 1 else 0)



def test_prefix_hit_leaves_the_rest_to_prefill():
    T.check_remainder_after_hit(BlockManager)
