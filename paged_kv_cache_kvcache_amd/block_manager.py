"""Python face of the native block manager (``pa_bm_*`` in libpa).

``BlockManager`` mirrors the allocator interface of the engine pages:
``can_allocate``, ``allocate``, ``deallocate``, ``can_append``,
``may_append`` and ``hash_blocks``, over caller-held sequence objects with
``token_ids`` (list of ints), ``block_table`` (list of ints),
``num_cached_tokens`` and ``block_size``. Every call crosses into the C++
allocator; this module only converts lists to arrays.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import binding as _b


def _i64(tokens) -> np.ndarray:
    return np.ascontiguousarray(tokens, dtype=np.int64)


def chained_hash(token_ids, prefix: int | None) -> int:
    t = _i64(token_ids)
    return int(_b.load().pa_bm_chained_hash(t.ctypes.data, len(t), 0 if prefix is None else prefix,
                                            0 if prefix is None else 1))


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _b.load()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise _b.PAError(_b.PA_ERR_INVALID_ARG, self._lib.pa_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def _check(self, rc):
        return _b._check(rc)

    def can_allocate(self, seq) -> int:
        """Cached leading blocks, or -1 when the prompt does not fit."""
        t = _i64(seq.token_ids)
        k = ctypes.c_int32()
        fits = self._check(self._lib.pa_bm_can_allocate(self._h, t.ctypes.data, len(t),
                                                        ctypes.byref(k)))
        return k.value if fits else -1

    def allocate(self, seq, num_cached_blocks: int) -> None:
        if seq.block_table:
            raise ValueError("sequence already holds blocks")
        t = _i64(seq.token_ids)
        cap = -(-len(t) // self.block_size)
        table = np.empty(max(cap, 1), dtype=np.int32)
        n = self._check(self._lib.pa_bm_allocate(self._h, t.ctypes.data, len(t),
                                                 int(num_cached_blocks), table.ctypes.data, cap))
        seq.block_table[:] = table[:n].tolist()
        seq.num_cached_tokens = int(num_cached_blocks) * self.block_size

    def deallocate(self, seq) -> None:
        table = np.ascontiguousarray(seq.block_table, dtype=np.int32)
        self._check(self._lib.pa_bm_deallocate(self._h, table.ctypes.data, len(table)))
        seq.num_cached_tokens = 0
        seq.block_table.clear()

    def can_append(self, seq) -> bool:
        return bool(self._check(self._lib.pa_bm_can_append(self._h, len(seq.token_ids))))

    def may_append(self, seq) -> None:
        n = len(seq.block_table)
        table = np.empty(n + 1, dtype=np.int32)
        table[:n] = seq.block_table
        m = self._check(self._lib.pa_bm_may_append(self._h, len(seq.token_ids), table.ctypes.data,
                                                   n, n + 1))
        if m > n:
            seq.block_table.append(int(table[n]))

    def hash_blocks(self, seq, num_scheduled_tokens: int) -> int:
        t = _i64(seq.token_ids)
        table = np.ascontiguousarray(seq.block_table, dtype=np.int32)
        return self._check(self._lib.pa_bm_hash_blocks(
            self._h, t.ctypes.data, len(t), table.ctypes.data, len(table),
            int(seq.num_cached_tokens), int(num_scheduled_tokens)))

    def state(self) -> dict:
        lib = self._lib
        nfree = self._check(lib.pa_bm_num_free(self._h))
        free = np.empty(max(nfree, 1), dtype=np.int32)
        lib.pa_bm_free_list(self._h, free.ctypes.data, nfree)
        ref, hashes = [], []
        rc, hv, hd = ctypes.c_int32(), ctypes.c_uint64(), ctypes.c_int32()
        for b in range(self.num_blocks):
            self._check(lib.pa_bm_block_state(self._h, b, ctypes.byref(rc), ctypes.byref(hv),
                                              ctypes.byref(hd)))
            ref.append(rc.value)
            hashes.append(hv.value if hd.value else None)
        n = self._check(lib.pa_bm_index_entries(self._h, None, None, 0))
        hk = np.empty(max(n, 1), dtype=np.uint64)
        hb = np.empty(max(n, 1), dtype=np.int32)
        lib.pa_bm_index_entries(self._h, hk.ctypes.data, hb.ctypes.data, n)
        return {"free": free[:nfree].tolist(), "used": [b for b in range(self.num_blocks) if ref[b] > 0],
                "ref_count": ref, "hash": hashes,
                "index": {int(k): int(v) for k, v in zip(hk[:n], hb[:n])}}
