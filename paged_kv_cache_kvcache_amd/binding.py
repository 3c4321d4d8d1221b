"""Thin ctypes binding of libpa (include/pa.h).

Argument marshalling only: shapes, strides and raw pointers are taken from
torch tensors (device memory) and numpy arrays (host metadata), and every
step of the hot path runs in the library's HIP kernels on torch's current
stream. There is no fallback: if ``libpa.so`` is missing the first call
raises ``LibraryNotBuilt``; a nonzero status raises ``PAError``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4

# Every symbol include/pa.h declares (checked by the CPU test suite).
EXPORTS = (
    "pa_store_kv", "pa_decode_workspace_size", "pa_decode", "pa_decode_partitioned",
    "pa_decode_step", "pa_mixed_varlen", "pa_mixed_workspace_size",
    "pa_decode_workspace_size_ex", "pa_prefill_varlen", "pa_build_metadata",
    "pa_last_error", "pa_version", "pa_set_debug",
    "pa_bm_create", "pa_bm_destroy", "pa_bm_chained_hash", "pa_bm_can_allocate", "pa_bm_allocate",
    "pa_bm_deallocate", "pa_bm_can_append", "pa_bm_may_append", "pa_bm_hash_blocks",
    "pa_bm_num_free", "pa_bm_free_list", "pa_bm_block_state", "pa_bm_lookup",
    "pa_bm_index_entries", "pa_decode_noalloc",
)


class LibraryNotBuilt(RuntimeError):
    pass


class PAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libpa error %d: %s" % (code, msg))
        self.code = code


class PaDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64)]


_LIB = None


def lib_path() -> str:
    return os.environ.get("PA_LIB", os.path.join(HERE, "libpa.so"))


def load():
    """Load libpa.so (once) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise LibraryNotBuilt("%s is not built; run `python -m paged_kv_cache_kvcache_amd.build` "
                              "(or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    pdesc = ctypes.POINTER(PaDesc)
    lib.pa_store_kv.argtypes = [vp, i64, vp, i64, vp, vp, vp, i32, pdesc, vp]
    lib.pa_store_kv.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [pdesc, i32, i32]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode_workspace_size_ex.argtypes = [pdesc, i32, i32, i32]
    lib.pa_decode_workspace_size_ex.restype = sz
    lib.pa_decode.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, f32, vp, vp, sz, pdesc, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, f32, vp, pdesc, vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_partitioned.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, f32, vp, vp, sz, i32,
                                          pdesc, vp]
    lib.pa_decode_partitioned.restype = ctypes.c_int
    lib.pa_decode_step.argtypes = [vp, vp, i64, vp, i64, vp, vp, vp, vp, i32, vp, i32, i32, f32, vp,
                                   vp, sz, pdesc, vp]
    lib.pa_decode_step.restype = ctypes.c_int
    lib.pa_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, f32, vp, pdesc,
                                      vp]
    lib.pa_prefill_varlen.restype = ctypes.c_int
    lib.pa_mixed_workspace_size.argtypes = [pdesc, i32, i32]
    lib.pa_mixed_workspace_size.restype = sz
    lib.pa_mixed_varlen.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp,
                                    sz, pdesc, vp]
    lib.pa_mixed_varlen.restype = ctypes.c_int
    lib.pa_build_metadata.argtypes = [vp, i32, vp, vp, i32, i32, vp, i64, vp, vp]
    lib.pa_build_metadata.restype = ctypes.c_int64
    u64 = ctypes.c_uint64
    lib.pa_bm_create.argtypes = [i32, i32]
    lib.pa_bm_create.restype = vp
    lib.pa_bm_destroy.argtypes = [vp]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_chained_hash.argtypes = [vp, i32, u64, i32]
    lib.pa_bm_chained_hash.restype = u64
    for name, args in (("pa_bm_can_allocate", [vp, vp, i32, vp]),
                       ("pa_bm_allocate", [vp, vp, i32, i32, vp, i32]),
                       ("pa_bm_deallocate", [vp, vp, i32]),
                       ("pa_bm_can_append", [vp, i32]),
                       ("pa_bm_may_append", [vp, i32, vp, i32, i32]),
                       ("pa_bm_hash_blocks", [vp, vp, i32, vp, i32, i32, i32]),
                       ("pa_bm_num_free", [vp]),
                       ("pa_bm_free_list", [vp, vp, i32]),
                       ("pa_bm_block_state", [vp, i32, vp, vp, vp]),
                       ("pa_bm_lookup", [vp, u64]),
                       ("pa_bm_index_entries", [vp, vp, vp, i32])):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = i32
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    lib.pa_set_debug.argtypes = [ctypes.c_int]
    lib.pa_set_debug.restype = ctypes.c_int
    _LIB = lib
    return lib


def pa_set_debug(on: bool) -> bool:
    """Debug mode on or off (device-resident preconditions checked before
    every launch); returns the previous setting."""
    return bool(load().pa_set_debug(1 if on else 0))


def _check(rc: int) -> int:
    if rc < 0:
        raise PAError(rc, load().pa_last_error().decode(errors="replace"))
    return rc


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("device tensor expected, got %s" % t.device)


def _desc_from_cache(k_cache, num_q_heads: int | None = None) -> PaDesc:
    if k_cache.dim() != 4:
        raise ValueError("cache must be [num_blocks, block_size, num_kv_heads, head_dim]")
    n, bsz, h_kv, d = k_cache.shape
    return PaDesc(int(num_q_heads if num_q_heads is not None else h_kv), int(h_kv), int(d),
                  int(bsz), int(n))


def _check_cache_pair(k_cache, v_cache):
    import torch
    for c in (k_cache, v_cache):
        if c.dtype != torch.bfloat16 or not c.is_contiguous():
            raise ValueError("caches must be contiguous bf16")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")


def pa_store_kv(k, v, k_cache, v_cache, slot_mapping, n_tokens: int | None = None) -> None:
    """Scatter ``k``/``v`` ``[n, H_kv, d]`` rows into the caches at
    ``slot_mapping`` (int32, -1 = skip). ``k``/``v`` may be row-strided views."""
    import torch
    _need_cuda(k, v, k_cache, v_cache, slot_mapping)
    _check_cache_pair(k_cache, v_cache)
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("k and v must be bf16")
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int32")
    n = int(k.shape[0]) if n_tokens is None else int(n_tokens)
    h_kv, d = k_cache.shape[2], k_cache.shape[3]
    for t in (k, v):
        if t.dim() != 3 or tuple(t.shape[1:]) != (h_kv, d):
            raise ValueError("k/v must be [n, H_kv, d] matching the cache")
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("k/v need contiguous heads (stride(-1) == 1, stride(1) == head_dim)")
    if slot_mapping.numel() < n or k.shape[0] < n or v.shape[0] < n:
        raise ValueError("fewer rows than n_tokens")
    desc = _desc_from_cache(k_cache)
    _check(load().pa_store_kv(k.data_ptr(), k.stride(0), v.data_ptr(), v.stride(0),
                              k_cache.data_ptr(), v_cache.data_ptr(), slot_mapping.data_ptr(), n,
                              ctypes.byref(desc), _stream(k_cache)))


def pa_decode_workspace_size(num_q_heads: int, k_cache, num_seqs: int, max_context_len: int,
                             partition_blocks: int = 0) -> int:
    desc = _desc_from_cache(k_cache, num_q_heads)
    return int(load().pa_decode_workspace_size_ex(ctypes.byref(desc), int(num_seqs),
                                                  int(max_context_len), int(partition_blocks)))


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
              max_context_len: int | None = None, workspace=None,
              partition_blocks: int = 0) -> None:
    """Paged decode: ``q`` ``[batch, H_q, d]`` -> ``out`` (same shape).

    ``max_context_len`` is a host bound on ``context_lens`` (defaults to the
    table width times the block size, so no device read is needed).
    """
    import torch
    _need_cuda(q, k_cache, v_cache, block_tables, context_lens, out)
    _check_cache_pair(k_cache, v_cache)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bf16")
    if not (q.is_contiguous() and out.is_contiguous() and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("q, out, block_tables and context_lens must be contiguous")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    batch, h_q, d = q.shape
    if tuple(out.shape) != (batch, h_q, d) or d != k_cache.shape[3]:
        raise ValueError("shape mismatch between q, out and the cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or context_lens.numel() != batch:
        raise ValueError("block_tables must be [batch, max_blocks], context_lens [batch]")
    max_blocks = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = max_blocks * int(k_cache.shape[1])
    desc = _desc_from_cache(k_cache, h_q)
    lib = load()
    need = int(lib.pa_decode_workspace_size_ex(ctypes.byref(desc), batch, int(max_context_len),
                                               int(partition_blocks)))
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            max_blocks, context_lens.data_ptr(), batch, int(max_context_len), float(scale),
            out.data_ptr(), ws_ptr, ws_bytes)
    if partition_blocks:
        _check(lib.pa_decode_partitioned(*args, int(partition_blocks), ctypes.byref(desc),
                                         _stream(q)))
    else:  # the library's partition choice: the plain entry point
        _check(lib.pa_decode(*args, ctypes.byref(desc), _stream(q)))


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                      max_context_len: int | None = None) -> None:
    """pa_decode with the library's own device scratch array as workspace
    (nothing is allocated; overlapping calls on one GPU race)."""
    import torch
    _need_cuda(q, k_cache, v_cache, block_tables, context_lens, out)
    _check_cache_pair(k_cache, v_cache)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bf16")
    if not (q.is_contiguous() and out.is_contiguous() and block_tables.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("q, out, block_tables and context_lens must be contiguous")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    batch, h_q, d = q.shape
    if tuple(out.shape) != (batch, h_q, d) or d != k_cache.shape[3]:
        raise ValueError("shape mismatch between q, out and the cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or context_lens.numel() != batch:
        raise ValueError("block_tables must be [batch, max_blocks], context_lens [batch]")
    max_blocks = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = max_blocks * int(k_cache.shape[1])
    desc = _desc_from_cache(k_cache, h_q)
    _check(load().pa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    block_tables.data_ptr(), max_blocks, context_lens.data_ptr(),
                                    batch, int(max_context_len), float(scale), out.data_ptr(),
                                    ctypes.byref(desc), _stream(q)))


def pa_decode_step(q, k_new, v_new, k_cache, v_cache, slot_mapping, block_tables, context_lens,
                   scale: float, out, max_context_len: int | None = None, workspace=None) -> None:
    """Fused store of each sequence's newest token (``k_new``/``v_new``
    ``[batch, H_kv, d]``, row-strided views allowed) + paged decode."""
    import torch
    _need_cuda(q, k_new, v_new, k_cache, v_cache, slot_mapping, block_tables, context_lens, out)
    _check_cache_pair(k_cache, v_cache)
    for t in (q, k_new, v_new, out):
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k_new, v_new and out must be bf16")
    for t in (slot_mapping, block_tables, context_lens):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("slot_mapping, block_tables and context_lens must be contiguous int32")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    batch, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    for t in (k_new, v_new):
        if t.dim() != 3 or tuple(t.shape) != (batch, h_kv, d) or t.stride(2) != 1 \
                or t.stride(1) != d:
            raise ValueError("k_new/v_new must be [batch, H_kv, d] with contiguous heads")
    if tuple(out.shape) != (batch, h_q, d) or slot_mapping.numel() != batch:
        raise ValueError("out must match q; slot_mapping must be [batch]")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or context_lens.numel() != batch:
        raise ValueError("block_tables must be [batch, max_blocks], context_lens [batch]")
    max_blocks = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = max_blocks * int(k_cache.shape[1])
    desc = _desc_from_cache(k_cache, h_q)
    lib = load()
    need = int(lib.pa_decode_workspace_size(ctypes.byref(desc), batch, int(max_context_len)))
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_step(q.data_ptr(), k_new.data_ptr(), k_new.stride(0), v_new.data_ptr(),
                              v_new.stride(0), k_cache.data_ptr(), v_cache.data_ptr(),
                              slot_mapping.data_ptr(), block_tables.data_ptr(), max_blocks,
                              context_lens.data_ptr(), batch, int(max_context_len), float(scale),
                              out.data_ptr(), ws_ptr, ws_bytes, ctypes.byref(desc), _stream(q)))


def pa_prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                      max_seqlen_k: int, block_tables, scale: float, out) -> None:
    """Varlen causal prefill over paged K/V: ``q``/``out`` ``[total_q, H_q, d]``."""
    import torch
    _need_cuda(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, out)
    _check_cache_pair(k_cache, v_cache)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bf16")
    for t in (cu_seqlens_q, cu_seqlens_k, block_tables):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("metadata must be contiguous int32")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    total_q, h_q, d = q.shape
    if tuple(out.shape) != (total_q, h_q, d) or d != k_cache.shape[3]:
        raise ValueError("shape mismatch between q, out and the cache")
    num_seqs = int(cu_seqlens_q.numel()) - 1
    if num_seqs < 0 or cu_seqlens_k.numel() != num_seqs + 1 or block_tables.shape[0] != num_seqs:
        raise ValueError("cu_seqlens must be [batch+1] and block_tables [batch, max_blocks]")
    desc = _desc_from_cache(k_cache, h_q)
    _check(load().pa_prefill_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), num_seqs,
                                    int(max_seqlen_q), int(max_seqlen_k), block_tables.data_ptr(),
                                    int(block_tables.shape[1]), float(scale), out.data_ptr(),
                                    ctypes.byref(desc), _stream(q)))


def pa_mixed_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, num_decode_rows: int,
                    max_seqlen_q: int, max_seqlen_k: int, block_tables, scale: float, out,
                    workspace=None) -> None:
    """Varlen step whose first ``num_decode_rows`` sequences have one query
    each (decode rows, run by the split-K decode kernels) followed by prefill
    rows (run by the MFMA prefill kernel)."""
    import torch
    _need_cuda(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, out)
    _check_cache_pair(k_cache, v_cache)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bf16")
    for t in (cu_seqlens_q, cu_seqlens_k, block_tables):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("metadata must be contiguous int32")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    total_q, h_q, d = q.shape
    if tuple(out.shape) != (total_q, h_q, d) or d != k_cache.shape[3]:
        raise ValueError("shape mismatch between q, out and the cache")
    num_seqs = int(cu_seqlens_q.numel()) - 1
    if num_seqs < 0 or cu_seqlens_k.numel() != num_seqs + 1 or block_tables.shape[0] != num_seqs:
        raise ValueError("cu_seqlens must be [batch+1] and block_tables [batch, max_blocks]")
    desc = _desc_from_cache(k_cache, h_q)
    lib = load()
    need = int(lib.pa_mixed_workspace_size(ctypes.byref(desc), int(num_decode_rows),
                                           int(max_seqlen_k)))
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_mixed_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                               cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), num_seqs,
                               int(num_decode_rows), int(max_seqlen_q), int(max_seqlen_k),
                               block_tables.data_ptr(), int(block_tables.shape[1]), float(scale),
                               out.data_ptr(), ws_ptr, ws_bytes, ctypes.byref(desc), _stream(q)))


def pa_build_metadata(block_tables: np.ndarray, starts, ends, block_size: int):
    """Host metadata of a step: ``(slot_mapping, cu_seqlens_q, cu_seqlens_k)``
    as int32 numpy arrays (runs in the library, on the CPU)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    if bt.ndim != 2:
        raise ValueError("block_tables must be 2-D")
    s = np.ascontiguousarray(starts, dtype=np.int32)
    e = np.ascontiguousarray(ends, dtype=np.int32)
    n = len(s)
    if len(e) != n or bt.shape[0] != n:
        raise ValueError("length mismatch")
    cap = int(np.maximum(e.astype(np.int64) - s, 0).sum())
    slots = np.empty(max(cap, 1), dtype=np.int32)
    cu_q = np.empty(n + 1, dtype=np.int32)
    cu_k = np.empty(n + 1, dtype=np.int32)
    got = _check(load().pa_build_metadata(bt.ctypes.data, bt.shape[1], s.ctypes.data,
                                          e.ctypes.data, n, int(block_size), slots.ctypes.data,
                                          cap, cu_q.ctypes.data, cu_k.ctypes.data))
    return slots[:got], cu_q, cu_k
