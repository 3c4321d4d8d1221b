"""Reference BlockManager: block pool, reference counts and chained-hash
prefix cache, in plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring). The product's native
allocator (``csrc/block_manager.cpp``) is checked against this module.

It follows "12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.8, and the
worked trace of "对照 Nano-vLLM 实现：读懂 vLLM 调度", §1.2. The state is:
  * per block: reference count, prefix hash (None = not hashed), token ids;
  * a FIFO of free block ids (taken from the front, returned to the back);
  * the set of used block ids (exactly the blocks with ref_count > 0);
  * a map from prefix hash to block id (the prefix-cache index).
A block's hash covers the whole prefix up to and including the block: it
hashes the previous block's hash (8 bytes, little endian; nothing for the
first block) followed by the block's token ids as int64 little endian, with
xxh64 (seed 0). Only full blocks are hashed. Freeing a block keeps its hash
and its index entry, so a later request can revive it; the stale entry is
dropped only when the block is handed out again.

Sequences are plain objects held by the caller: ``token_ids`` (the whole
sequence so far), ``block_table`` and ``num_cached_tokens``.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np
import xxhash


def chained_hash(token_ids, prefix: int | None) -> int:
    """xxh64 of (prefix hash as 8 little-endian bytes, if any) + the tokens as
    int64 little-endian bytes ([P1 §12.8] compute_hash)."""
    h = xxhash.xxh64(seed=0)
    if prefix is not None:
        h.update(int(prefix).to_bytes(8, "little"))
    h.update(np.asarray(token_ids, dtype="<i8").tobytes())
    return h.intdigest()


@dataclass
class Seq:
    token_ids: list
    block_size: int
    block_table: list = field(default_factory=list)
    num_cached_tokens: int = 0

    def __len__(self):
        return len(self.token_ids)

    @property
    def num_blocks(self) -> int:
        return -(-len(self.token_ids) // self.block_size)

    def block(self, i: int) -> list:
        return self.token_ids[i * self.block_size:(i + 1) * self.block_size]


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.ref_count = [0] * num_blocks
        self.hash: list = [None] * num_blocks
        self.tokens: list = [[] for _ in range(num_blocks)]
        self.free = deque(range(num_blocks))
        self.used: set = set()
        self.index: dict = {}

    # -- single blocks --------------------------------------------------
    def _take_free_block(self) -> int:
        """Hand out the block at the front of the free FIFO; drop its stale
        index entry if the index still points at it; reset it (count 1, no
        hash, no tokens)."""
        bid = self.free.popleft()
        assert self.ref_count[bid] == 0
        old = self.hash[bid]
        if old is not None and self.index.get(old) == bid:
            del self.index[old]
        self.ref_count[bid] = 1
        self.hash[bid] = None
        self.tokens[bid] = []
        self.used.add(bid)
        return bid

    def _release_block(self, bid: int) -> None:
        """Return an unreferenced block to the back of the FIFO, keeping its
        hash and index entry."""
        assert self.ref_count[bid] == 0
        self.used.remove(bid)
        self.free.append(bid)

    # -- prefill ----------------------------------------------------------
    def _cached_prefix(self, seq: Seq):
        """Walk the full blocks except the last: count leading blocks whose
        chained hash is indexed and whose stored tokens match (collision
        guard). Returns (hits, how many of them are in use right now)."""
        h = None
        hits, in_use = 0, 0
        for i in range(seq.num_blocks - 1):
            toks = seq.block(i)
            h = chained_hash(toks, h)
            bid = self.index.get(h)
            if bid is None or self.tokens[bid] != list(toks):
                break
            hits += 1
            if bid in self.used:
                in_use += 1
        return hits, in_use

    def can_allocate(self, seq: Seq) -> int:
        """Number of leading cached blocks, or -1 if the free pool cannot
        hold the blocks that are neither cached-and-in-use nor free-revivable
        (a cached block that sits in the free pool still takes a free slot)."""
        hits, in_use = self._cached_prefix(seq)
        need = seq.num_blocks - in_use
        if len(self.free) < need:
            return -1
        return hits

    def allocate(self, seq: Seq, num_cached_blocks: int) -> None:
        assert not seq.block_table
        h = None
        for i in range(num_cached_blocks):
            h = chained_hash(seq.block(i), h)
            bid = self.index[h]
            if bid in self.used:
                self.ref_count[bid] += 1
            else:  # freed but not yet reused: revive it
                self.ref_count[bid] = 1
                self.free.remove(bid)
                self.used.add(bid)
            seq.block_table.append(bid)
        for _ in range(num_cached_blocks, seq.num_blocks):
            seq.block_table.append(self._take_free_block())
        seq.num_cached_tokens = num_cached_blocks * self.block_size

    def deallocate(self, seq: Seq) -> None:
        for bid in reversed(seq.block_table):
            self.ref_count[bid] -= 1
            if self.ref_count[bid] == 0:
                self._release_block(bid)
        seq.num_cached_tokens = 0
        seq.block_table.clear()

    # -- decode -----------------------------------------------------------
    def can_append(self, seq: Seq) -> bool:
        """A sequence whose length is 1 more than a multiple of the block
        size has just spilled into a new block and needs one free block."""
        return len(self.free) >= (1 if len(seq) % self.block_size == 1 else 0)

    def may_append(self, seq: Seq) -> None:
        if len(seq) % self.block_size == 1:
            seq.block_table.append(self._take_free_block())

    # -- after a step ---------------------------------------------------------
    def hash_blocks(self, seq: Seq, num_scheduled_tokens: int) -> None:
        """Hash and index the blocks that the step filled: those wholly
        inside [0, num_cached_tokens + num_scheduled_tokens) and not inside
        [0, num_cached_tokens)."""
        bs = self.block_size
        start = seq.num_cached_tokens // bs
        end = (seq.num_cached_tokens + num_scheduled_tokens) // bs
        if start == end:
            return
        h = self.hash[seq.block_table[start - 1]] if start > 0 else None
        for i in range(start, end):
            bid = seq.block_table[i]
            toks = seq.block(i)
            h = chained_hash(toks, h)
            self.hash[bid] = h
            self.tokens[bid] = list(toks)
            self.index[h] = bid

    # -- inspection -------------------------------------------------------------
    def state(self) -> dict:
        return {"free": list(self.free), "used": sorted(self.used),
                "ref_count": list(self.ref_count), "hash": list(self.hash),
                "index": dict(self.index)}
