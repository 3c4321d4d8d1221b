"""fp64 oracle: address mapping, KV store, paged decode and varlen prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the CPU-baseline leg of the benchmark use this module.

Pages cited (titles as published; sections as numbered on each page):
  [P1] "12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.6 (Attention layer:
       paged KV cache), §12.7 (ModelRunner: prepare_prefill / prepare_decode),
       §12.8 (BlockManager: can_append / may_append).
  [P2] kyonqi, "nano-vllm 05" (ModelRunner): prepare_prefill, prepare_decode,
       prepare_block_tables.
  [P4] "vLLM 深度解读", §3 (PagedAttention CUDA kernel).
  [P5] "Nano-vLLM 源码解读 - 3. PagedAttention", §3 (physical blocks vs
       logical sequence: the two-step mapping) and §4 (slot_mapping; its
       prefill and decode paths).

Conventions (the readings of the pages are listed in the design doc):
  * a cache is ``[num_blocks, block_size, num_kv_heads, head_dim]`` bf16 bits
    (uint16); a slot is a row index into the cache viewed as
    ``[num_blocks * block_size, num_kv_heads, head_dim]``;
  * q-head ``h`` reads kv-head ``h // G`` with ``G = num_q_heads // num_kv_heads``;
  * a prefill query ``i`` of a sequence with ``q_len`` queries and ``k_len``
    keys sits at absolute position ``k_len - q_len + i`` and sees keys
    ``0 .. k_len - q_len + i`` (causal, aligned to the end);
  * a sequence with no keys has an all-zero output.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 input

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly.

    A bf16 value is the upper half of the float32 with the same sign,
    exponent and leading mantissa bits, so shifting the pattern into the high
    16 bits of a 32-bit word gives that float32 exactly; float32 -> float64
    is exact as well.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------- address mapping

def slot_of(block_table, position: int, block_size: int) -> int:
    """Pool row that holds token ``position`` of a sequence.

    [P5 §3]: the logical block ``position // block_size`` is translated to a
    physical block through the sequence's block table; the token sits at
    offset ``position % block_size`` inside it, and the physical block starts
    at row ``block_id * block_size`` of the pool.  [P1 §12.6] states the same
    formula for the store kernel's slot_mapping.
    """
    logical_block = position // block_size
    physical_block = int(block_table[logical_block])
    if physical_block < 0:
        raise ValueError("position %d maps to a padding table entry" % position)
    return physical_block * block_size + position % block_size


def slots_for_range(block_table, start: int, end: int, block_size: int) -> list[int]:
    """Slots of the tokens at positions ``start .. end-1`` of one sequence.

    [P5 §4, prefill path]: a step computes K/V for a contiguous range of
    positions (the uncached part of the prompt, or one chunk of it); each
    token is written at the slot the two-step mapping gives for its position.
    The page's loop walks the blocks from ``start // B`` to ``ceil(end / B)``
    and clips the first and the last one; listing the positions one by one
    is the same set in the same order.
    """
    if not 0 <= start <= end:
        raise ValueError("need 0 <= start <= end")
    return [slot_of(block_table, p, block_size) for p in range(start, end)]


def decode_slot(block_table, seq_len: int, block_size: int) -> int:
    """Slot of the newest token of a sequence of ``seq_len`` tokens.

    [P5 §4, decode path] and [P1 §12.7 prepare_decode]: one new token per
    sequence, at position ``seq_len - 1``.
    """
    if seq_len <= 0:
        raise ValueError("decode needs at least one token")
    return slot_of(block_table, seq_len - 1, block_size)


def cu_seqlens(lengths) -> list[int]:
    """Running totals ``[0, l0, l0+l1, ...]`` that mark where each sequence of
    a packed varlen batch starts and ends ([P1 §12.6], the cu_seqlens
    explanation under the FlashAttention argument notes)."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


def build_metadata(block_tables: np.ndarray, starts, ends, block_size: int):
    """Host-side metadata of one step, [P5 §4] / [P2 prepare_prefill].

    Sequence ``b`` computes positions ``starts[b] .. ends[b]-1`` and attends
    over keys ``0 .. ends[b]-1``. Returns ``(slot_mapping, cu_seqlens_q,
    cu_seqlens_k)`` as int32 arrays: queries are packed in batch order,
    ``cu_seqlens_q`` accumulates ``end - start`` and ``cu_seqlens_k``
    accumulates ``end`` (the cached prefix counts as keys).
    """
    slots: list[int] = []
    for b, (s, e) in enumerate(zip(starts, ends)):
        slots.extend(slots_for_range(block_tables[b], int(s), int(e), block_size))
    cu_q = cu_seqlens([int(e) - int(s) for s, e in zip(starts, ends)])
    cu_k = cu_seqlens([int(e) for e in ends])
    return (np.asarray(slots, dtype=np.int32), np.asarray(cu_q, dtype=np.int32),
            np.asarray(cu_k, dtype=np.int32))


# ---------------------------------------------------------------- KV store

def store_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
             slot_mapping) -> tuple[np.ndarray, np.ndarray]:
    """Return copies of the caches with token ``i``'s K/V written at row
    ``slot_mapping[i]``.

    [P1 §12.6, store kernel]: one token per program; a slot of -1 marks a
    padding entry and is skipped; the token's ``num_kv_heads * head_dim``
    values are copied unchanged (a bit copy: no arithmetic touches them).
    Rows that no slot names are left as they were.
    """
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    n_blocks, bsz, h_kv, d = kc.shape
    k_rows = kc.reshape(n_blocks * bsz, h_kv, d)
    v_rows = vc.reshape(n_blocks * bsz, h_kv, d)
    k = np.asarray(k, dtype=np.uint16)
    v = np.asarray(v, dtype=np.uint16)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        if not 0 <= slot < n_blocks * bsz:
            raise ValueError("slot %d outside the pool" % slot)
        k_rows[slot] = k[i]
        v_rows[slot] = v[i]
    return kc, vc


def gather_rows(cache: np.ndarray, block_table, n_tokens: int) -> np.ndarray:
    """Rows ``slot_of(t)`` for ``t < n_tokens``, as float64 ``[n, H_kv, d]``.

    The logical view a sequence has of its paged K (or V): the tokens in
    position order, fetched through the block table ([P5 §3]; [P4 §3] reads
    K the same way inside its kernel sketch).
    """
    n_blocks, bsz, h_kv, d = cache.shape
    rows = cache.reshape(n_blocks * bsz, h_kv, d)
    idx = [slot_of(block_table, t, bsz) for t in range(n_tokens)]
    return bf16_bits_to_f64(rows[np.asarray(idx, dtype=np.int64)]) if idx else \
        np.zeros((0, h_kv, d), dtype=np.float64)


def used_rows(block_tables: np.ndarray, n_tokens, block_size: int) -> np.ndarray:
    """Sorted unique slots that hold tokens ``0 .. n_tokens[b]-1`` of some
    sequence ``b``; every other pool row is unused (test helper)."""
    s: set[int] = set()
    for b, n in enumerate(np.asarray(n_tokens).tolist()):
        s.update(slot_of(block_tables[b], t, block_size) for t in range(int(n)))
    return np.asarray(sorted(s), dtype=np.int64)


# --------------------------------------------------------------- attention

def _softmax_attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys @ q) @ values for one query vector (float64)."""
    s = scale * (keys @ q)
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ values


def decode_one(q_b: np.ndarray, k_cache, v_cache, block_table, ctx: int, scale: float) -> np.ndarray:
    """Decode attention of one sequence: ``q_b`` is ``[H_q, d]`` bf16 bits.

    [P1 §12.6, decode branch; P4 §3]: the single new query of each q-head
    attends over all ``ctx`` tokens of the sequence (the newest one
    included, which is why the store runs first), K and V read through the
    block table. The causal flag passed on that page changes nothing for a
    single query placed after every key.
    """
    h_q, d = q_b.shape
    h_kv = k_cache.shape[2]
    group = h_q // h_kv
    if ctx == 0:
        return np.zeros((h_q, d), dtype=np.float64)
    keys = gather_rows(k_cache, block_table, ctx)
    vals = gather_rows(v_cache, block_table, ctx)
    qf = bf16_bits_to_f64(q_b)
    out = np.empty((h_q, d), dtype=np.float64)
    for h in range(h_q):
        g = h // group
        out[h] = _softmax_attend(qf[h], keys[:, g, :], vals[:, g, :], scale)
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, rows=None) -> np.ndarray:
    """Paged decode for a batch; ``q`` is ``[batch, H_q, d]`` bf16 bits.

    Returns float64 ``[batch, H_q, d]``. ``rows`` restricts the work to a
    subset of sequences (others are left as zeros).
    """
    q = np.asarray(q, dtype=np.uint16)
    batch, h_q, d = q.shape
    out = np.zeros((batch, h_q, d), dtype=np.float64)
    todo = range(batch) if rows is None else rows
    for b in todo:
        out[b] = decode_one(q[b], k_cache, v_cache, block_tables[b], int(context_lens[b]), scale)
    return out


def prefill_one(q_seq: np.ndarray, k_cache, v_cache, block_table, k_len: int, scale: float,
                query_rows=None) -> np.ndarray:
    """Causal attention of one sequence's ``q_len`` queries over ``k_len``
    paged keys; ``q_seq`` is ``[q_len, H_q, d]`` bf16 bits.

    [P1 §12.6, prefill branch with prefix cache]: the new tokens are stored
    first, then keys and values, cached prefix and new suffix alike, are
    read from the cache through the block table. Query ``i`` is the token at
    position ``k_len - q_len + i`` and sees keys at positions up to its own.
    """
    q_len, h_q, d = q_seq.shape
    if q_len > k_len:
        raise ValueError("q_len > k_len")
    h_kv = k_cache.shape[2]
    group = h_q // h_kv
    offset = k_len - q_len
    keys = gather_rows(k_cache, block_table, k_len)
    vals = gather_rows(v_cache, block_table, k_len)
    qf = bf16_bits_to_f64(q_seq)
    out = np.zeros((q_len, h_q, d), dtype=np.float64)
    todo = range(q_len) if query_rows is None else query_rows
    for i in todo:
        visible = offset + i + 1
        for h in range(h_q):
            g = h // group
            out[i, h] = _softmax_attend(qf[i, h], keys[:visible, g, :], vals[:visible, g, :], scale)
    return out


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, scale: float,
                   seqs=None) -> np.ndarray:
    """Varlen causal prefill over a packed batch; ``q`` is ``[total_q, H_q, d]``.

    [P1 §12.6, flash_attn_varlen_func notes]: sequences are packed along the
    token axis and delimited by cu_seqlens; q and k lengths differ when a
    prefix is cached. Returns float64 ``[total_q, H_q, d]``; ``seqs``
    restricts the work to a subset of sequences.
    """
    q = np.asarray(q, dtype=np.uint16)
    out = np.zeros(q.shape, dtype=np.float64)
    n = len(cu_seqlens_q) - 1
    todo = range(n) if seqs is None else seqs
    for b in todo:
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k_len = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        out[q0:q1] = prefill_one(q[q0:q1], k_cache, v_cache, block_tables[b], k_len, scale)
    return out
