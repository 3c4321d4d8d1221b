"""Reference block allocator with a chained-hash prefix cache, in plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring). The product's native
allocator (``csrc/block_manager.cpp``) is checked against this module.

What it models ("12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.8, the
block manager's behaviour; "对照 Nano-vLLM 实现：读懂 vLLM 调度", §1.2, the
worked trace that pins it), written as a state and the rules that every
operation keeps, not as a transcription of the page's code:

State
  * ``holders[b]``: how many live sequences have block ``b`` in their table
    (the reference count; 0 for a free block).
  * ``free_order``: the free blocks, in the order they became free (all
    blocks, ascending, at the start). Fresh blocks are taken from its front.
  * ``content[b]``: for a block that was filled and hashed, the pair
    (prefix hash, token ids); absent otherwise.
  * ``lookup``: prefix hash -> block, the cache index.

Rules
  R1 (prefix hash) The hash of block i of a token sequence covers the whole
     prefix: xxh64 (seed 0) over the hash of block i-1 as 8 little-endian
     bytes (nothing for block 0) followed by block i's token ids as int64
     little endian. Only full blocks are hashed.
  R2 (cache hit) A prompt's cached prefix is the longest run of leading
     blocks, never including its last block, whose prefix hashes are in
     ``lookup`` with stored tokens equal to the prompt's (a hash collision
     is not a hit).
  R3 (admission) A prompt fits when the free pool holds one block for every
     block of the prompt that is not a hit held by a live sequence (a hit
     that sits in the free pool still uses a free slot: it is taken out).
  R4 (allocation) The table is the hit blocks, in order (each held once
     more; a free one leaves the free pool), followed by fresh blocks from
     the front of ``free_order``. A fresh block loses its old content and,
     if ``lookup`` still names it, that index entry.
  R5 (release) A finished sequence lets go of its blocks last to first;
     each block nobody holds any more joins the back of ``free_order``,
     keeping its content and index entry (a later prompt may revive it).
  R6 (growth) A decoding sequence whose length is one past a multiple of the
     block size has spilled into a new block: one fresh block (R4) is
     appended, and admission requires one free block.
  R7 (hashing) After a step, every block that the computed tokens have now
     filled, and that was not full before the step, gets its prefix hash
     and tokens recorded, and ``lookup`` maps that hash to it.

Sequences are plain objects held by the caller: ``token_ids`` (the whole
sequence so far), ``block_table`` and ``num_cached_tokens``. The method
names are the page's (they are the interface the trace drives).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from itertools import takewhile

import numpy as np
import xxhash


def chained_hash(token_ids, prefix: int | None) -> int:
    """R1 for one block: xxh64 of (prefix hash as 8 little-endian bytes, if
    any) + the tokens as int64 little-endian bytes."""
    data = b"" if prefix is None else int(prefix).to_bytes(8, "little")
    data += np.asarray(token_ids, dtype="<i8").tobytes()
    return xxhash.xxh64_intdigest(data, seed=0)


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


def prefix_hashes(seq: Seq, n_blocks: int) -> list:
    """R1 over the first n_blocks blocks of a sequence."""
    out, h = [], None
    for i in range(n_blocks):
        h = chained_hash(seq.block(i), h)
        out.append(h)
    return out


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.holders = [0] * num_blocks
        self.free_order = list(range(num_blocks))
        self.content: dict = {}
        self.lookup: dict = {}

    # -- R2 / R3 -------------------------------------------------------------
    def _hits(self, seq: Seq) -> list:
        """Blocks of the cached prefix (R2), in order."""
        candidates = prefix_hashes(seq, seq.num_blocks - 1)

        def hit(i_h):
            i, h = i_h
            b = self.lookup.get(h)
            return b is not None and self.content[b][1] == list(seq.block(i))
        return [self.lookup[h] for _, h in takewhile(hit, enumerate(candidates))]

    def can_allocate(self, seq: Seq) -> int:
        """Number of cached leading blocks, or -1 if the prompt does not fit
        (R3)."""
        hits = self._hits(seq)
        held = sum(1 for b in hits if self.holders[b] > 0)
        return len(hits) if len(self.free_order) >= seq.num_blocks - held else -1

    # -- R4 ------------------------------------------------------------------
    def _fresh(self) -> int:
        b = self.free_order.pop(0)
        old = self.content.pop(b, None)
        if old is not None and self.lookup.get(old[0]) == b:
            del self.lookup[old[0]]
        self.holders[b] = 1
        return b

    def allocate(self, seq: Seq, num_cached_blocks: int) -> None:
        assert not seq.block_table
        hits = self._hits(seq)[:num_cached_blocks]
        assert len(hits) == num_cached_blocks
        for b in hits:
            if self.holders[b] == 0:
                self.free_order.remove(b)  # revived from the free pool
            self.holders[b] += 1
        seq.block_table = hits + [self._fresh() for _ in range(seq.num_blocks - len(hits))]
        seq.num_cached_tokens = num_cached_blocks * self.block_size

    # -- R5 ------------------------------------------------------------------
    def deallocate(self, seq: Seq) -> None:
        for b in seq.block_table[::-1]:
            self.holders[b] -= 1
            if self.holders[b] == 0:
                self.free_order.append(b)
        seq.block_table.clear()
        seq.num_cached_tokens = 0

    # -- R6 ------------------------------------------------------------------
    def _spilled(self, seq: Seq) -> bool:
        return len(seq) % self.block_size == 1

    def can_append(self, seq: Seq) -> bool:
        return len(self.free_order) >= int(self._spilled(seq))

    def may_append(self, seq: Seq) -> None:
        if self._spilled(seq):
            seq.block_table.append(self._fresh())

    # -- R7 ------------------------------------------------------------------
    def hash_blocks(self, seq: Seq, num_scheduled_tokens: int) -> None:
        bs = self.block_size
        full_before = seq.num_cached_tokens // bs
        full_after = (seq.num_cached_tokens + num_scheduled_tokens) // bs
        hashes = prefix_hashes(seq, full_after)
        for i in range(full_before, full_after):
            b = seq.block_table[i]
            self.content[b] = (hashes[i], list(seq.block(i)))
            self.lookup[hashes[i]] = b

    # -- inspection ------------------------------------------------------------
    def state(self) -> dict:
        return {"free": list(self.free_order),
                "used": [b for b, n in enumerate(self.holders) if n > 0],
                "ref_count": list(self.holders),
                "hash": [self.content[b][0] if b in self.content else None
                         for b in range(len(self.holders))],
                "index": dict(self.lookup)}
