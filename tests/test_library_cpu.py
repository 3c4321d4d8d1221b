"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, rejects bad arguments on the host, and its host metadata builder
(slot_mapping, cu_seqlens) agrees bit for bit with the oracle."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
from paged_kv_cache_kvcache_amd import binding as B
from paged_kv_cache_kvcache_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.fail("libpa.so is not built: run __graft_entry__.build()")
    return B.load()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for required in ("pa_store_kv", "pa_decode", "pa_prefill_varlen"):
        assert required in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.pa_version().decode().count(".") == 2


def _desc(h_q=32, h_kv=8, d=128, bsz=256, n=10):
    return B.PaDesc(h_q, h_kv, d, bsz, n)


def test_host_argument_checks_need_no_gpu(lib):
    d = _desc()
    assert lib.pa_store_kv(None, 0, None, 0, None, None, None, 0, ctypes.byref(d), None) == 0
    assert lib.pa_store_kv(None, 0, None, 0, None, None, None, 4, ctypes.byref(d), None) == \
        B.PA_ERR_INVALID_ARG
    assert lib.pa_store_kv(None, 0, None, 0, None, None, None, 4, None, None) == B.PA_ERR_INVALID_ARG
    bad = _desc(h_q=30)
    assert lib.pa_decode(None, None, None, None, 0, None, 1, 0, 1.0, None, None, 0,
                         ctypes.byref(bad), None) == B.PA_ERR_INVALID_ARG
    assert b"multiple" in lib.pa_last_error()
    for kw in (dict(d=96), dict(bsz=8), dict(bsz=48), dict(bsz=2048), dict(h_q=64, h_kv=2),
               dict(h_q=34, h_kv=2), dict(h_q=34, h_kv=2, d=64)):  # group sizes 32, 17
        assert lib.pa_decode(None, None, None, None, 0, None, 1, 0, 1.0, None, None, 0,
                             ctypes.byref(_desc(**kw)), None) == B.PA_ERR_UNSUPPORTED
    for bsz in (16, 32, 64, 128, 512, 1024):  # every built block size: an empty batch is a no-op
        assert lib.pa_decode(None, None, None, None, 0, None, 0, 0, 1.0, None, None, 0,
                             ctypes.byref(_desc(bsz=bsz)), None) == 0
    for h_q, h_kv in ((8, 8), (16, 8), (32, 8), (64, 8), (64, 4), (24, 8), (40, 8), (28, 4),
                      (24, 2)):  # group sizes 1 .. 16, powers of two or not
        for d_ in (64, 128):
            assert lib.pa_decode(None, None, None, None, 0, None, 0, 0, 1.0, None, None, 0,
                                 ctypes.byref(_desc(h_q=h_q, h_kv=h_kv, d=d_)), None) == 0
    assert lib.pa_decode(None, None, None, None, 0, None, 0, 0, 1.0, None, None, 0,
                         ctypes.byref(d), None) == 0  # empty batch: no-op
    # workspace checked before any launch
    # Every plan starts with a fixed 256 KiB header of arrival counters (one
    # int32 per (sequence, kv-head) of a stream-grid call), then its partials.
    HDR = 65536 * 4
    # explicit partitions (the partitioned grid): one partial (o[d], m, l)
    # fp32 per (sequence, q-head, partition) when some sequence needs > 1
    # partition; nothing (not even the header) when none does
    for pb in (1, 2, 3):
        parts = -(-4096 // (256 * pb))
        assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 4, 4096, pb) == \
            HDR + 4 * 32 * parts * (128 + 2) * 4
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 4, 256, 1) == 0
    # more work items (sequence x pair of kv-heads x partition) than the 256
    # CUs: the partials plus one int32 dispatch rank per (sequence,
    # partition), 16-byte rounded, and 16 bytes for the partition length the
    # order kernel chooses, up to 4096 sequences
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 256, 8192, 1) == \
        HDR + 256 * 32 * 32 * (128 + 2) * 4 + 256 * 32 * 4 + 16
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 4096, 256, 1) == HDR + 4096 * 4 + 16
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 4097, 256, 1) == 0
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 64, 256, 1) == 0  # 256 items
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 65, 256, 1) == HDR + 65 * 4 + 12 + 16
    # the library's choice (the stream grid): W grabs per kv-head group,
    # W = 1,024 waves / (waves per grab x groups); one partial row per grab
    # and sequence boundary, (W + num_seqs - 1) rows of H_q (o[d], m, l),
    # whatever the context length
    for ns, ctx in ((4, 256), (4, 4096), (256, 8192), (4096, 256)):
        # 32 q / 8 kv heads, d 128: waves of two kv-heads, 4 groups -> W 256
        assert lib.pa_decode_workspace_size(ctypes.byref(d), ns, ctx) == \
            HDR + (256 + ns - 1) * 32 * (128 + 2) * 4
    g8 = _desc(h_q=64, h_kv=8)  # matrix-core grabs: 2 waves, 4 groups -> W 128
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(g8), 64, 8192, 0) == \
        HDR + (128 + 63) * 64 * (128 + 2) * 4
    small = _desc(h_q=4, h_kv=2, d=64)  # one kv-head per wave: W 512
    assert lib.pa_decode_workspace_size(ctypes.byref(small), 4, 300) == \
        HDR + (512 + 3) * 4 * (64 + 2) * 4
    # the header holds 65,536 (sequence, kv-head) counters: more pairs take
    # the partitioned grid
    assert lib.pa_decode_workspace_size(ctypes.byref(d), 8192, 256) == \
        HDR + (256 + 8191) * 32 * (128 + 2) * 4
    big = lib.pa_decode_workspace_size(ctypes.byref(d), 8193, 256)
    assert big == 0  # 8,193 x 8 pairs: partitioned, one partition each, no ordering
    # an explicit partition length is kept: 2 partitions of 4,096
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(g8), 64, 8192, 16) == \
        HDR + 64 * 64 * 2 * (128 + 2) * 4 + 64 * 2 * 4 + 16
    need = lib.pa_decode_workspace_size(ctypes.byref(d), 4, 4096)
    assert need > 0
    fake = ctypes.c_void_p(0x1000)
    assert lib.pa_decode(fake, fake, fake, fake, 16, fake, 4, 4096, 1.0, fake, None, 0,
                         ctypes.byref(d), None) == B.PA_ERR_WORKSPACE
    assert lib.pa_decode(fake, fake, fake, fake, 4, fake, 4, 4096, 1.0, fake, None, 0,
                         ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG  # table too narrow


def test_metadata_golden_examples(lib):
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "slot_mapping_examples.json")))
    for ex in gold["range_examples"]:
        slots, cu_q, cu_k = B.pa_build_metadata(np.array([ex["block_table"]]), [ex["start"]],
                                                [ex["end"]], ex["block_size"])
        assert slots.tolist() == ex["slot_mapping"], ex["cite"]
    for ex in gold["cu_seqlens_examples"]:
        n = len(ex["lengths"])
        tables = np.zeros((n, 1), dtype=np.int32)
        _, cu_q, _ = B.pa_build_metadata(tables, [0] * n, ex["lengths"], 1 << 20)
        assert cu_q.tolist() == ex["cu_seqlens"]


@pytest.mark.parametrize("name", ["tiny", "qwen3-0.6b", "prefill"])
def test_metadata_matches_oracle_on_workloads(lib, name):
    case = W.make_case(name, threads=4)
    if isinstance(case, W.DecodeCase):
        starts, ends = case.starts, case.context_lens
    else:
        starts, ends = case.starts, case.ends
    got = B.pa_build_metadata(case.block_tables, starts, ends, case.block_size)
    ref = oracle.build_metadata(case.block_tables, starts, ends, case.block_size)
    for g, r in zip(got, ref):
        assert g.dtype == np.int32 and np.array_equal(g, r)


def test_metadata_matches_oracle_random(lib):
    rng = np.random.default_rng(99)
    for _ in range(50):
        bsz = int(rng.choice([4, 16, 256]))
        n = int(rng.integers(1, 9))
        ends = rng.integers(0, 6 * bsz, size=n)
        starts = (ends * rng.random(n)).astype(np.int64)
        width = max(1, int(-(-ends.max() // bsz)))
        tables = rng.permutation(n * width + 7)[: n * width].reshape(n, width).astype(np.int32)
        got = B.pa_build_metadata(tables, starts, ends, bsz)
        ref = oracle.build_metadata(tables, starts, ends, bsz)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)


def test_metadata_rejects_padding_and_bad_ranges(lib):
    tables = np.array([[3, -1]], dtype=np.int32)
    with pytest.raises(B.PAError):
        B.pa_build_metadata(tables, [0], [300], 256)  # position 256 hits -1 padding
    with pytest.raises(B.PAError):
        B.pa_build_metadata(tables, [5], [2], 256)
    with pytest.raises(B.PAError):
        B.pa_build_metadata(tables, [0], [600], 256)  # needs 3 blocks, table has 2


def test_debug_switch_needs_no_gpu(lib):
    prev = lib.pa_set_debug(1)
    try:
        assert lib.pa_set_debug(1) == 1
        d = _desc()
        # host checks and no-op calls come first: nothing reaches the device
        assert lib.pa_store_kv(None, 0, None, 0, None, None, None, 0, ctypes.byref(d), None) == 0
        assert lib.pa_store_kv(None, 0, None, 0, None, None, None, 4, ctypes.byref(d), None) == \
            B.PA_ERR_INVALID_ARG
        assert lib.pa_decode(None, None, None, None, 0, None, 0, 0, 1.0, None, None, 0,
                             ctypes.byref(d), None) == 0
        assert lib.pa_set_debug(0) == 1
        assert lib.pa_set_debug(0) == 0
    finally:
        lib.pa_set_debug(prev)


def test_scale_must_be_positive_and_finite(lib):
    """The kernels scale the maximum of the raw scores, which is the maximum
    of the scaled scores only for scale > 0: every attention entry point
    rejects other scales on the host, before touching any pointer."""
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    for bad in (0.0, -0.125, float("nan"), float("inf"), -float("inf")):
        assert lib.pa_decode(fake, fake, fake, fake, 16, fake, 4, 4096, bad, fake, None, 0,
                             ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG
        assert b"scale" in lib.pa_last_error()
        assert lib.pa_decode_partitioned(fake, fake, fake, fake, 16, fake, 4, 4096, bad, fake,
                                         None, 0, 2, ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG
        assert lib.pa_decode_step(fake, fake, 1024, fake, 1024, fake, fake, fake, fake, 16, fake,
                                  4, 4096, bad, fake, None, 0, ctypes.byref(d),
                                  None) == B.PA_ERR_INVALID_ARG
        assert lib.pa_prefill_varlen(fake, fake, fake, fake, fake, 4, 100, 4096, fake, 16, bad,
                                     fake, ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG
        assert b"scale" in lib.pa_last_error()
        assert lib.pa_mixed_varlen(fake, fake, fake, fake, fake, 4, 2, 100, 4096, fake, 16, bad,
                                   fake, None, 0, ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG
    # a positive scale passes that check (and then fails on the missing workspace)
    assert lib.pa_decode(fake, fake, fake, fake, 16, fake, 4, 4096, 0.125, fake, None, 0,
                         ctypes.byref(d), None) == B.PA_ERR_WORKSPACE


def test_long_partitions_are_cut_to_the_longest_context(lib):
    """An explicit partition longer than ceil(max_context_len / 256) units
    holds every sequence whole: the workspace equals that of the cut length
    (no partials; the dispatch order, if any, has one entry per sequence),
    however large the request, and a context above 2^30 is refused."""
    d = _desc()
    for pb in (32, 127, 128, 200, 255, 256, 4096, 2 ** 31 - 1):
        for seqs, ctx in ((4, 8192), (65, 8192), (256, 16384)):
            whole = -(-ctx // 256)
            assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), seqs, ctx, pb) == \
                lib.pa_decode_workspace_size_ex(ctypes.byref(d), seqs, ctx, min(pb, whole))
    assert lib.pa_decode_workspace_size_ex(ctypes.byref(d), 65, 8192, 200) == \
        65536 * 4 + 65 * 4 + 12 + 16
    fake = ctypes.c_void_p(0x1000)
    assert lib.pa_decode(fake, fake, fake, fake, 2 ** 22 + 1, fake, 4, 2 ** 30 + 1, 0.125, fake,
                         None, 0, ctypes.byref(_desc(bsz=1024)), None) == B.PA_ERR_INVALID_ARG
    assert b"max_context_len" in lib.pa_last_error()


def test_noalloc_refuses_batches_beyond_its_scratch_before_any_device_call(lib):
    """pa_decode_noalloc's workspace is the library's 64 MiB device array: a
    batch that needs more is refused on the host (no GPU needed to see it),
    after the usual argument checks."""
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    need = lib.pa_decode_workspace_size(ctypes.byref(d), 4096, 16384)
    assert need > 64 << 20
    assert lib.pa_decode_noalloc(fake, fake, fake, fake, 64, fake, 4096, 16384, 0.125, fake,
                                 ctypes.byref(d), None) == B.PA_ERR_WORKSPACE
    msg = lib.pa_last_error().decode()
    assert "pa_decode_noalloc" in msg and str(need) in msg and str(64 << 20) in msg
    assert lib.pa_decode_noalloc(fake, fake, fake, fake, 64, fake, 4096, 16384, -1.0, fake,
                                 ctypes.byref(d), None) == B.PA_ERR_INVALID_ARG
    assert lib.pa_decode_noalloc(None, None, None, None, 0, None, 0, 0, 1.0, None,
                                 ctypes.byref(d), None) == 0  # empty batch: no-op
    # the Qwen3-8B decode batch fits
    assert lib.pa_decode_workspace_size(ctypes.byref(d), 256, 8192) <= 64 << 20
