"""Seeded synthetic inputs for the paged KV-cache hot path.

This module only draws inputs: random bf16 tensors, sequence lengths and
block tables (a random permutation of the physical pool handed out to the
sequences in order). It holds none of the method's arithmetic: slot
addresses, cu_seqlens and attention are computed by the library (and,
independently, by the oracle in the tests).

Recipe (the same for every consumer; see the design doc for the table):
  * a named case with seed ``S`` draws its random sequence lengths from
    ``numpy.random.default_rng(S)``; everything else comes from
    ``default_rng(S + 1)`` in the order: block permutation -> q -> new-token
    K -> new-token V;
  * the pool contents are filled chunk by chunk, chunk ``c`` of cache ``s``
    (0 = K, 1 = V) from ``default_rng([S + 1, 1000 + s, c])`` so that large
    pools can be filled by several threads and still come out identical;
  * every value is N(0, 1) drawn in float32 and rounded to bf16 with
    round-to-nearest-even; tensors hold bf16 bit patterns as uint16;
  * "uniform in [a, b]" lengths are integers with both ends included;
  * a pool holds the blocks the sequences need plus 10% free blocks
    (rounded up) unless the case fixes its size;
  * a sequence of n tokens holds ceil(n / block_size) blocks; block-table
    rows are padded with -1.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 256
_CHUNK = 1 << 22  # elements per independently seeded pool chunk


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Inputs here are finite normal draws, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return round_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _fill_chunk(flat: np.ndarray, seed: int, stream: int, c: int) -> None:
    lo = c * _CHUNK
    hi = min(flat.size, lo + _CHUNK)
    rng = np.random.default_rng([seed, 1000 + stream, c])
    flat[lo:hi] = round_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))


def pool_bf16(num_blocks: int, block_size: int, h_kv: int, d: int, seed: int, stream: int,
              threads: int | None = None) -> np.ndarray:
    """A ``[num_blocks, block_size, h_kv, d]`` pool of N(0,1) bf16 bits."""
    out = np.empty((num_blocks, block_size, h_kv, d), dtype=np.uint16)
    flat = out.reshape(-1)
    n_chunks = max(1, math.ceil(flat.size / _CHUNK))
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            _fill_chunk(flat, seed, stream, c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda c: _fill_chunk(flat, seed, stream, c), range(n_chunks)))
    return out


def blocks_needed(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(n_tokens) // block_size)


def pad_tables(tables: list[list[int]]) -> np.ndarray:
    width = max(1, max((len(t) for t in tables), default=1))
    out = np.full((len(tables), width), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        out[b, :len(t)] = t
    return out


@dataclass
class DecodeCase:
    """One decode step: every sequence adds one token (K/V in ``k_new``/``v_new``)
    at position ``context_lens[b] - 1`` and attends over ``context_lens[b]``
    tokens. ``context_lens[b] == 0`` marks a padding row (no token, no blocks)."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q: np.ndarray             # [batch, H_q, d] bf16 bits
    k_new: np.ndarray         # [batch, H_kv, d]
    v_new: np.ndarray
    k_cache: np.ndarray       # [N, B, H_kv, d]
    v_cache: np.ndarray
    block_tables: np.ndarray  # [batch, max_blocks] int32, -1 padded
    context_lens: np.ndarray  # [batch] int32
    scale: float
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def starts(self) -> np.ndarray:
        """First position computed this step (the newest token); 0 for padding rows."""
        return np.maximum(self.context_lens - 1, 0).astype(np.int32)


@dataclass
class PrefillCase:
    """One prefill step: sequence ``b`` computes positions
    ``starts[b] .. ends[b]-1`` (queries packed in batch order) over keys
    ``0 .. ends[b]-1``; positions below ``starts[b]`` are already cached."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q: np.ndarray             # [total_q, H_q, d]
    k_new: np.ndarray         # [total_q, H_kv, d]
    v_new: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    starts: np.ndarray        # [batch] int32
    ends: np.ndarray          # [batch] int32
    scale: float
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.starts.shape[0])


def decode_case(num_q_heads: int, num_kv_heads: int, head_dim: int, context_lens,
                seed: int, num_blocks: int | None = None, block_size: int = BLOCK_SIZE,
                name: str = "custom", threads: int | None = None) -> DecodeCase:
    """Decode inputs for the given lengths (already drawn by the caller)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    need = [blocks_needed(n, block_size) for n in ctx.tolist()]
    total = sum(need)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.1 * total))
    if num_blocks < total:
        raise ValueError("pool of %d blocks cannot hold %d" % (num_blocks, total))
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables, pos = [], 0
    for n in need:
        tables.append(perm[pos:pos + n].tolist())
        pos += n
    batch = len(ctx)
    q = normal_bf16(rng, (batch, num_q_heads, head_dim))
    k_new = normal_bf16(rng, (batch, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (batch, num_kv_heads, head_dim))
    k_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 0, threads)
    v_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 1, threads)
    return DecodeCase(name, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      q, k_new, v_new, k_cache, v_cache, pad_tables(tables), ctx,
                      1.0 / math.sqrt(head_dim), seed)


def prefill_case(num_q_heads: int, num_kv_heads: int, head_dim: int, prefix_len: int,
                 suffix_lens, seed: int, num_blocks: int | None = None,
                 block_size: int = BLOCK_SIZE, name: str = "custom",
                 threads: int | None = None, share_prefix: bool = True) -> PrefillCase:
    """Prefill inputs: every sequence has ``prefix_len`` cached tokens (held in
    the same physical blocks by all sequences when ``share_prefix``; the
    prefix must then be whole blocks) followed by its own uncached suffix."""
    rng = np.random.default_rng(seed)
    suffix = np.asarray(suffix_lens, dtype=np.int32)
    batch = len(suffix)
    ends = (prefix_len + suffix).astype(np.int32)
    starts = np.full(batch, prefix_len, dtype=np.int32)
    if share_prefix:
        if prefix_len % block_size:
            raise ValueError("a shared prefix must be whole blocks")
        n_prefix = prefix_len // block_size
        own = [blocks_needed(e, block_size) - n_prefix for e in ends.tolist()]
        total = n_prefix + sum(own)
    else:
        n_prefix = 0
        own = [blocks_needed(e, block_size) for e in ends.tolist()]
        total = sum(own)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.1 * total))
    if num_blocks < total:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    shared = perm[:n_prefix].tolist()
    pos = n_prefix
    tables = []
    for n in own:
        tables.append(shared + perm[pos:pos + n].tolist())
        pos += n
    total_q = int(suffix.sum())
    q = normal_bf16(rng, (total_q, num_q_heads, head_dim))
    k_new = normal_bf16(rng, (total_q, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (total_q, num_kv_heads, head_dim))
    k_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 0, threads)
    v_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 1, threads)
    return PrefillCase(name, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       q, k_new, v_new, k_cache, v_cache, pad_tables(tables), starts, ends,
                       1.0 / math.sqrt(head_dim), seed,
                       {"prefix_len": prefix_len, "shared_prefix_blocks": shared})


def mixed_case(num_q_heads: int, num_kv_heads: int, head_dim: int, decode_lens, chunks,
               seed: int, block_size: int = BLOCK_SIZE, name: str = "mixed",
               threads: int | None = None) -> PrefillCase:
    """One mixed step: decode rows (one new token at position len-1 of a
    sequence of ``len`` tokens) followed by chunked-prefill rows, each given
    as ``(cached, chunk)``: positions ``cached .. cached+chunk-1`` are new
    (``cached`` need not be block-aligned). Every sequence owns its blocks,
    which cover all ``end`` positions."""
    rng = np.random.default_rng(seed)
    starts, ends = [], []
    for n in decode_lens:
        starts.append(int(n) - 1)
        ends.append(int(n))
    for cached, chunk in chunks:
        starts.append(int(cached))
        ends.append(int(cached) + int(chunk))
    starts = np.asarray(starts, dtype=np.int32)
    ends = np.asarray(ends, dtype=np.int32)
    need = [blocks_needed(e, block_size) for e in ends.tolist()]
    num_blocks = max(1, math.ceil(1.1 * sum(need)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables, pos = [], 0
    for n in need:
        tables.append(perm[pos:pos + n].tolist())
        pos += n
    total_q = int((ends - starts).sum())
    q = normal_bf16(rng, (total_q, num_q_heads, head_dim))
    k_new = normal_bf16(rng, (total_q, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (total_q, num_kv_heads, head_dim))
    k_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 0, threads)
    v_cache = pool_bf16(num_blocks, block_size, num_kv_heads, head_dim, seed, 1, threads)
    return PrefillCase(name, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       q, k_new, v_new, k_cache, v_cache, pad_tables(tables), starts, ends,
                       1.0 / math.sqrt(head_dim), seed,
                       {"decode_rows": len(decode_lens), "prefill_rows": len(chunks)})


# ------------------------------------------------------------ named workloads

SEEDS = {"tiny": 1001, "qwen3-0.6b": 1002, "qwen3-8b": 1003, "long": 1004, "prefill": 1005,
         "mixed": 1006, "gqa8": 1007, "gqa16": 1008, "skewed": 1009}

DESCRIPTIONS = {
    "tiny": "decode, 4 q / 2 kv heads, d 64, B 256, pool 16, ctx {1,17,256,300}",
    "qwen3-0.6b": "decode, 16 q / 8 kv heads, d 128, B 256, 64 seqs, ctx U[128,4096]",
    "qwen3-8b": "decode, 32 q / 8 kv heads, d 128, B 256, 256 seqs, ctx U[512,8192]",
    "long": "decode, 32 q / 8 kv heads, d 128, B 256, 32 seqs at ctx 16384",
    "prefill": "varlen causal prefill, 32 q / 8 kv heads, d 128, B 256, 16 prompts: "
               "shared 1024-token prefix + suffix U[100,2000]",
    "mixed": "mixed varlen step, 32 q / 8 kv heads, d 128, B 256: 224 decode rows "
             "(ctx U[512,8192]) + 4 chunked-prefill rows of 512 tokens starting mid-block "
             "(cached U[100,4000])",
    # larger GQA groups than the pages' shapes, same batch and lengths as
    # qwen3-8b: 8 and 16 q-heads per kv-head
    "gqa8": "decode, 64 q / 8 kv heads, d 128, B 256, 256 seqs, ctx U[512,8192]",
    "gqa16": "decode, 64 q / 4 kv heads, d 128, B 256, 256 seqs, ctx U[512,8192]",
    # one long context among short ones: the split-K partition and the grid's
    # balance under the most uneven length mix of a decode batch
    "skewed": "decode, 32 q / 8 kv heads, d 128, B 256, 256 seqs: 1 at ctx 8192 + 255 at 100",
}


def make_case(name: str, seed: int | None = None, threads: int | None = None,
              block_size: int = BLOCK_SIZE):
    """The named workloads (lengths drawn first from the case's rng). Another
    block size keeps every length and draw; only the pool's shape, the tables
    and (for "tiny") the pool size change."""
    seed = SEEDS[name] if seed is None else seed
    kw = dict(name=name, threads=threads, block_size=block_size)
    if name == "tiny":
        return decode_case(4, 2, 64, [1, 17, 256, 300], seed + 1,
                           num_blocks=16 if block_size == BLOCK_SIZE else None, **kw)
    if name == "qwen3-0.6b":
        ctx = np.random.default_rng(seed).integers(128, 4096 + 1, size=64)
        return decode_case(16, 8, 128, ctx, seed + 1, **kw)
    if name == "qwen3-8b":
        ctx = np.random.default_rng(seed).integers(512, 8192 + 1, size=256)
        return decode_case(32, 8, 128, ctx, seed + 1, **kw)
    if name == "long":
        return decode_case(32, 8, 128, [16384] * 32, seed + 1, **kw)
    if name == "skewed":
        return decode_case(32, 8, 128, [8192] + [100] * 255, seed + 1, **kw)
    if name in ("gqa8", "gqa16"):  # the qwen3-8b lengths, own contents
        ctx = np.random.default_rng(SEEDS["qwen3-8b"]).integers(512, 8192 + 1, size=256)
        return decode_case(64, 8 if name == "gqa8" else 4, 128, ctx, seed + 1, **kw)
    if name == "prefill":
        suffix = np.random.default_rng(seed).integers(100, 2000 + 1, size=16)
        return prefill_case(32, 8, 128, 1024, suffix, seed + 1, **kw)
    if name == "mixed":
        rng = np.random.default_rng(seed)
        dec = rng.integers(512, 8192 + 1, size=224)
        cached = rng.integers(100, 4000 + 1, size=4)
        return mixed_case(32, 8, 128, dec, [(int(c), 512) for c in cached], seed + 1, **kw)
    raise KeyError(name)
