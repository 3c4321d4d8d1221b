"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: the
worked examples printed on the pages (tests/golden/), a library routine
(torch's scaled_dot_product_attention in float64) on the special case that
reduces to it, closed forms, invariants, and a plain scalar evaluation on
tiny inputs. The last test plants plausible mistakes in copies of the oracle
functions and checks that the pins catch each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_kv_cache_kvcache_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def f64(bits):
    return oracle.bf16_bits_to_f64(bits)


# ------------------------------------------------------------------ address


def check_range_examples(slots_fn):
    for ex in _golden()["range_examples"]:
        got = slots_fn(ex["block_table"], ex["start"], ex["end"], ex["block_size"])
        assert list(got) == ex["slot_mapping"], ex["cite"]


def test_slot_examples_from_pages():
    check_range_examples(oracle.slots_for_range)


def test_cu_seqlens_example_from_pages():
    for ex in _golden()["cu_seqlens_examples"]:
        assert oracle.cu_seqlens(ex["lengths"]) == ex["cu_seqlens"], ex["cite"]


def test_block_boundary_example_from_pages():
    """The page's fact (a 256-token sequence fits one block, the 257th token
    starts the second) on a block table of the test's own choosing: the
    newest token lands in the last of the sequence's blocks, at the offset
    the fact implies (the last row of block 0; the first row of block 1)."""
    table = [5, 9]  # arbitrary physical blocks, not from the page
    for ex in _golden()["block_boundary_examples"]:
        bsz = ex["block_size"]
        for c in ex["cases"]:
            slot = oracle.decode_slot(table, c["seq_len"], bsz)
            block, offset = divmod(slot, bsz)
            assert block == table[c["blocks"] - 1], ex["cite"]
            assert offset == c["seq_len"] - 1 - (c["blocks"] - 1) * bsz, ex["cite"]
            assert (offset == bsz - 1) == (c["blocks"] == 1)


def _decode_slot_last_block_form(block_table, seq_len, block_size):
    # The decode pages write the newest token's slot as: last table entry *
    # block size + tokens held by the last block - 1.
    n_blocks = -(-seq_len // block_size)
    last_block_tokens = seq_len - (n_blocks - 1) * block_size
    return block_table[n_blocks - 1] * block_size + last_block_tokens - 1


def test_decode_slot_matches_last_block_formula():
    rng = np.random.default_rng(7)
    for _ in range(500):
        bsz = int(rng.choice([4, 16, 256]))
        n = int(rng.integers(1, 20 * bsz))
        table = rng.permutation(10_000)[: -(-n // bsz)].tolist()
        assert oracle.decode_slot(table, n, bsz) == _decode_slot_last_block_form(table, n, bsz)


def _prefill_slots_block_walk(block_table, start, end, bsz):
    # The prefill page's block walk with first/last-block clipping, written
    # as its prose describes it: blocks start//B .. ceil(end/B)-1; the first
    # begins at start % B, the last stops at end.
    out = []
    first, last = start // bsz, -(-end // bsz)
    for i in range(first, last):
        lo = block_table[i] * bsz + (start % bsz if i == first else 0)
        hi = block_table[i] * bsz + (bsz if i != last - 1 else end - i * bsz)
        out.extend(range(lo, hi))
    return out


def test_prefill_slots_match_block_walk():
    rng = np.random.default_rng(8)
    for _ in range(300):
        bsz = int(rng.choice([4, 16, 256]))
        end = int(rng.integers(1, 12 * bsz))
        start = int(rng.integers(0, end))
        table = rng.permutation(5000)[: -(-end // bsz)].tolist()
        assert oracle.slots_for_range(table, start, end, bsz) == \
            _prefill_slots_block_walk(table, start, end, bsz)


def test_build_metadata_packs_in_batch_order():
    tables = np.array([[3, 0], [1, -1], [2, 4]], dtype=np.int32)
    slots, cu_q, cu_k = oracle.build_metadata(tables, [2, 0, 5], [6, 3, 7], 4)
    assert cu_q.tolist() == [0, 4, 7, 9]
    assert cu_k.tolist() == [0, 6, 9, 16]
    assert slots.tolist() == [14, 15, 0, 1, 4, 5, 6, 17, 18]


# -------------------------------------------------------------------- store


def test_store_writes_named_rows_and_only_them():
    case = W.decode_case(4, 2, 64, [1, 17, 256, 300], seed=5, num_blocks=16)
    slots = [oracle.decode_slot(case.block_tables[b], int(n), 256)
             for b, n in enumerate(case.context_lens)]
    slots[2] = -1  # a padding entry is skipped
    kc, vc = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    rows_k = kc.reshape(-1, 2, 64)
    rows_k0 = case.k_cache.reshape(-1, 2, 64)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(rows_k[s], case.k_new[i])
            assert np.array_equal(vc.reshape(-1, 2, 64)[s], case.v_new[i])
    untouched = np.ones(rows_k.shape[0], bool)
    untouched[[s for s in slots if s >= 0]] = False
    assert np.array_equal(rows_k[untouched], rows_k0[untouched])
    assert np.array_equal(case.k_cache, rows_k0.reshape(case.k_cache.shape))  # input not mutated


def test_store_then_gather_returns_token():
    case = W.decode_case(8, 8, 128, [300, 5], seed=6)
    slots = [oracle.decode_slot(case.block_tables[b], int(n), 256)
             for b, n in enumerate(case.context_lens)]
    kc, _ = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    for b, n in enumerate(case.context_lens):
        rows = oracle.gather_rows(kc, case.block_tables[b], int(n))
        assert np.array_equal(rows[-1], f64(case.k_new[b]))


# ---------------------------------------------------------------- attention


def _identity_case(h_q, h_kv, d, lens, seed, bsz=256):
    """Sequence b's blocks are laid out consecutively in the pool, so its
    gathered K/V is a contiguous slice of the pool."""
    rng = np.random.default_rng(seed)
    need = [-(-n // bsz) for n in lens]
    nb = sum(need)
    kc = W.normal_bf16(rng, (nb, bsz, h_kv, d))
    vc = W.normal_bf16(rng, (nb, bsz, h_kv, d))
    tables, pos = [], 0
    for n in need:
        tables.append(list(range(pos, pos + n)))
        pos += n
    return kc, vc, W.pad_tables(tables)


def _contiguous(cache, table, n):
    nb = -(-n // cache.shape[1])
    blk = cache[table[0]:table[0] + nb]
    return f64(blk.reshape(-1, *cache.shape[2:])[:n])


def check_decode_vs_sdpa(decode_fn):
    """Identity table: paged decode == contiguous attention (library routine)."""
    for (h_q, h_kv, d, lens, seed) in [(4, 2, 64, [1, 17, 256, 300], 11),
                                       (8, 2, 128, [513, 40], 12),
                                       (6, 6, 32, [77], 13),
                                       (10, 2, 32, [40, 260], 14),    # group size 5
                                       (21, 3, 32, [300], 15)]:       # group size 7
        kc, vc, bt = _identity_case(h_q, h_kv, d, lens, seed)
        rng = np.random.default_rng(seed + 100)
        q = W.normal_bf16(rng, (len(lens), h_q, d))
        scale = 1.0 / math.sqrt(d)
        got = decode_fn(q, kc, vc, bt, np.asarray(lens, np.int32), scale)
        for b, n in enumerate(lens):
            K = torch.from_numpy(_contiguous(kc, bt[b], n)).permute(1, 0, 2)[None]
            V = torch.from_numpy(_contiguous(vc, bt[b], n)).permute(1, 0, 2)[None]
            Q = torch.from_numpy(f64(q[b]))[None, :, None, :]
            ref = F.scaled_dot_product_attention(Q, K, V, scale=scale, enable_gqa=True)
            np.testing.assert_allclose(got[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_decode_identity_table_equals_sdpa():
    check_decode_vs_sdpa(oracle.decode)


def check_prefill_vs_full_recompute(prefill_fn):
    """Prefix-cached prefill: suffix queries over cached + new keys give the
    suffix rows of full causal attention over the whole sequence (computed
    with the library routine, where q_len == k_len)."""
    for (h_q, h_kv, d, prefix, suffix, seed) in [(4, 2, 64, [256, 0, 300], [40, 5, 1], 21),
                                                 (8, 2, 128, [512], [300], 22),
                                                 (6, 2, 32, [100], [60], 23)]:  # group size 3
        ends = [p + s for p, s in zip(prefix, suffix)]
        kc, vc, bt = _identity_case(h_q, h_kv, d, ends, seed)
        rng = np.random.default_rng(seed + 100)
        full_q = [W.normal_bf16(rng, (e, h_q, d)) for e in ends]
        q = np.concatenate([fq[p:] for fq, p in zip(full_q, prefix)])
        cu_q = np.cumsum([0] + suffix).astype(np.int32)
        cu_k = np.cumsum([0] + ends).astype(np.int32)
        scale = 1.0 / math.sqrt(d)
        got = prefill_fn(q, kc, vc, cu_q, cu_k, bt, scale)
        for b, (p, e) in enumerate(zip(prefix, ends)):
            K = torch.from_numpy(_contiguous(kc, bt[b], e)).permute(1, 0, 2)[None]
            V = torch.from_numpy(_contiguous(vc, bt[b], e)).permute(1, 0, 2)[None]
            Q = torch.from_numpy(f64(full_q[b])).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(Q, K, V, scale=scale, is_causal=True,
                                                 enable_gqa=True)[0].permute(1, 0, 2)
            np.testing.assert_allclose(got[cu_q[b]:cu_q[b + 1]], ref[p:].numpy(),
                                       rtol=0, atol=1e-12)


def test_prefill_prefix_cache_equals_full_causal_recompute():
    check_prefill_vs_full_recompute(oracle.prefill_varlen)


def _permute_pool(case_kc, case_vc, tables, seed):
    rng = np.random.default_rng(seed)
    n = case_kc.shape[0]
    pi = rng.permutation(n)
    kc = np.empty_like(case_kc)
    vc = np.empty_like(case_vc)
    kc[pi] = case_kc
    vc[pi] = case_vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    return kc, vc, t2


def check_decode_permutation_invariance(decode_fn):
    case = W.decode_case(8, 2, 64, [1, 255, 256, 257, 700], seed=31)
    ref = decode_fn(case.q, case.k_cache, case.v_cache, case.block_tables,
                    case.context_lens, case.scale)
    kc, vc, bt = _permute_pool(case.k_cache, case.v_cache, case.block_tables, 32)
    got = decode_fn(case.q, kc, vc, bt, case.context_lens, case.scale)
    assert np.array_equal(got, ref)


def test_decode_invariant_under_block_permutation():
    check_decode_permutation_invariance(oracle.decode)


def test_prefill_invariant_under_block_permutation():
    case = W.prefill_case(4, 2, 64, 256, [30, 260], seed=33)
    _, cu_q, cu_k = oracle.build_metadata(case.block_tables, case.starts, case.ends, 256)
    ref = oracle.prefill_varlen(case.q, case.k_cache, case.v_cache, cu_q, cu_k,
                                case.block_tables, case.scale)
    kc, vc, bt = _permute_pool(case.k_cache, case.v_cache, case.block_tables, 34)
    got = oracle.prefill_varlen(case.q, kc, vc, cu_q, cu_k, bt, case.scale)
    assert np.array_equal(got, ref)


def check_single_token_is_value(decode_fn):
    """One key: softmax weight 1, so out = that token's V (exactly)."""
    case = W.decode_case(8, 2, 64, [1, 1, 1], seed=41)
    out = decode_fn(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                    case.scale)
    for b in range(3):
        v = f64(case.v_cache[case.block_tables[b, 0], 0])  # [H_kv, d]
        for h in range(8):
            assert np.array_equal(out[b, h], v[h // 4])


def test_ctx1_returns_value_exactly():
    check_single_token_is_value(oracle.decode)


def check_equal_keys_give_mean_value(decode_fn):
    """All keys equal: uniform weights, out = mean of V over the context,
    taken per kv-head, which also fixes which kv-head each q-head reads."""
    case = W.decode_case(8, 4, 32, [5, 300], seed=42)
    kc = case.k_cache.copy()
    kc[:] = kc[0, 0]  # every row holds the same K (per kv-head)
    out = decode_fn(case.q, kc, case.v_cache, case.block_tables, case.context_lens,
                    case.scale)
    for b, n in enumerate(case.context_lens):
        rows = []
        for t in range(int(n)):
            blk = case.block_tables[b, t // 256]
            rows.append(f64(case.v_cache[blk, t % 256]))
        mean = np.mean(rows, axis=0)
        for h in range(8):
            np.testing.assert_allclose(out[b, h], mean[h // 2], rtol=0, atol=1e-13)


def test_equal_keys_give_mean_of_values():
    check_equal_keys_give_mean_value(oracle.decode)


def test_empty_context_row_is_zero():
    case = W.decode_case(4, 2, 64, [0, 3], seed=43)
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                        case.context_lens, case.scale)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_decode_equals_prefill_with_one_query():
    case = W.decode_case(8, 2, 64, [1, 90, 511], seed=44)
    dec = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                        case.context_lens, case.scale)
    cu_q = np.arange(4, dtype=np.int32)
    cu_k = np.concatenate([[0], np.cumsum(case.context_lens)]).astype(np.int32)
    pre = oracle.prefill_varlen(case.q, case.k_cache, case.v_cache, cu_q, cu_k,
                                case.block_tables, case.scale)
    np.testing.assert_allclose(pre, dec, rtol=0, atol=1e-14)


def test_split_combine_equals_single_pass():
    """The decode kernels split a sequence into partitions and merge the
    per-partition (max, sum, unnormalised output) triples; in base 2:
    M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p 2^(m_p - M) / L.
    Written out here in fp64 over uneven splits, it must equal the oracle's
    single pass over the whole sequence."""
    case = W.decode_case(8, 2, 64, [1000], seed=46)
    ref = oracle.decode_one(case.q[0], case.k_cache, case.v_cache, case.block_tables[0], 1000,
                            case.scale)
    keys = oracle.gather_rows(case.k_cache, case.block_tables[0], 1000)
    vals = oracle.gather_rows(case.v_cache, case.block_tables[0], 1000)
    q = f64(case.q[0])
    c = case.scale / math.log(2.0)  # scores in log2 units
    for cuts in ([0, 1000], [0, 256, 1000], [0, 1, 2, 999, 1000], [0, 300, 301, 700, 1000]):
        for h in range(8):
            g = h // 4
            parts = []
            for lo, hi in zip(cuts[:-1], cuts[1:]):
                s2 = (keys[lo:hi, g, :] @ q[h]) * c
                m = s2.max()
                w = np.exp2(s2 - m)
                parts.append((m, w.sum(), w @ vals[lo:hi, g, :]))
            M = max(m for m, _, _ in parts)
            L = sum(l * 2.0 ** (m - M) for m, l, _ in parts)
            out = sum(o * 2.0 ** (m - M) for m, _, o in parts) / L
            np.testing.assert_allclose(out, ref[h], rtol=0, atol=1e-12)


def test_shared_prefix_rows_identical_across_sequences():
    """Sequences whose tables share the prefix blocks: prefix queries see only
    prefix keys (causality), so their outputs agree across sequences."""
    case = W.prefill_case(4, 2, 64, 512, [10, 300, 45], seed=45)
    # prefill every position (nothing cached): starts 0, the same shared q
    # rows for the prefix positions
    rng = np.random.default_rng(46)
    prefix_q = W.normal_bf16(rng, (512, 4, 64))
    qs, lens = [], []
    for b, e in enumerate(case.ends.tolist()):
        own = W.normal_bf16(rng, (e - 512, 4, 64))
        qs.append(np.concatenate([prefix_q, own]))
        lens.append(e)
    q = np.concatenate(qs)
    cu = np.cumsum([0] + lens).astype(np.int32)
    out = oracle.prefill_varlen(q, case.k_cache, case.v_cache, cu, cu, case.block_tables,
                                case.scale)
    first = out[cu[0]:cu[0] + 512]
    for b in range(1, 3):
        assert np.array_equal(out[cu[b]:cu[b] + 512], first)
    assert not np.array_equal(out[cu[1] + 512], out[cu[2] + 512])


def _scalar_attention(qv, keys, vals, scale):
    # log-sum-exp form evaluated with Python floats
    scores = [scale * math.fsum(a * b for a, b in zip(qv, k)) for k in keys]
    m = max(scores)
    lse = m + math.log(math.fsum(math.exp(s - m) for s in scores))
    w = [math.exp(s - lse) for s in scores]
    return [math.fsum(wi * v[e] for wi, v in zip(w, vals)) for e in range(len(qv))]


def test_tiny_prefill_matches_scalar_evaluation():
    """Tiny shapes, block size 4: every output element recomputed with
    Python floats directly from the pool layout [N, B, H_kv, d]."""
    bsz, h_q, h_kv, d = 4, 4, 2, 3
    rng = np.random.default_rng(51)
    nb = 6
    kc = W.normal_bf16(rng, (nb, bsz, h_kv, d))
    vc = W.normal_bf16(rng, (nb, bsz, h_kv, d))
    tables = np.array([[4, 1, 3], [0, 5, -1]], dtype=np.int32)
    ends = [9, 6]
    starts = [6, 0]
    qlens = [e - s for s, e in zip(starts, ends)]
    q = W.normal_bf16(rng, (sum(qlens), h_q, d))
    cu_q = np.cumsum([0] + qlens).astype(np.int32)
    cu_k = np.cumsum([0] + ends).astype(np.int32)
    got = oracle.prefill_varlen(q, kc, vc, cu_q, cu_k, tables, 0.7)
    kf, vf, qf = f64(kc), f64(vc), f64(q)
    for b in range(2):
        for i in range(qlens[b]):
            pos = starts[b] + i
            for h in range(h_q):
                g = h * h_kv // h_q
                keys = [kf[tables[b][t // bsz], t % bsz, g] for t in range(pos + 1)]
                vals = [vf[tables[b][t // bsz], t % bsz, g] for t in range(pos + 1)]
                ref = _scalar_attention(qf[cu_q[b] + i, h], keys, vals, 0.7)
                np.testing.assert_allclose(got[cu_q[b] + i, h], ref, rtol=0, atol=1e-13)


# ------------------------------------------------------ planted mistakes


def _mutant_decode(kind):
    def fn(q, kc, vc, bt, ctx, scale):
        q = np.asarray(q)
        batch, h_q, d = q.shape
        h_kv = kc.shape[2]
        group = h_q // h_kv
        out = np.zeros((batch, h_q, d))
        bsz = kc.shape[1]
        for b in range(batch):
            n = int(ctx[b])
            if kind == "drop_last_token":
                n -= 1
            if n <= 0:
                continue
            if kind == "logical_block_as_physical":
                idx = list(range(n))
            else:
                idx = [int(bt[b][t // bsz]) * bsz + t % bsz for t in range(n)]
            K = f64(kc.reshape(-1, h_kv, d)[idx])
            V = f64(vc.reshape(-1, h_kv, d)[idx])
            for h in range(h_q):
                g = h % h_kv if kind == "gqa_modulo" else h // group
                s = (scale if kind != "no_scale" else 1.0) * (K[:, g] @ f64(q[b, h]))
                p = np.exp(s - s.max())
                if kind != "unnormalised":
                    p /= p.sum()
                out[b, h] = p @ (K[:, g] if kind == "k_for_v" else V[:, g])
        return out
    return fn


def _mutant_prefill(kind):
    def fn(q, kc, vc, cu_q, cu_k, bt, scale):
        out = np.zeros(q.shape)
        h_q, d = q.shape[1:]
        h_kv = kc.shape[2]
        bsz = kc.shape[1]
        for b in range(len(cu_q) - 1):
            q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
            k_len = int(cu_k[b + 1] - cu_k[b])
            idx = [int(bt[b][t // bsz]) * bsz + t % bsz for t in range(k_len)]
            K = f64(kc.reshape(-1, h_kv, d)[idx])
            V = f64(vc.reshape(-1, h_kv, d)[idx])
            off = k_len - (q1 - q0)
            for i in range(q1 - q0):
                vis = (i + 1) if kind == "top_left_causal" else (off + i + 1)
                if kind == "strict_causal":
                    vis -= 1
                vis = max(vis, 1)
                for h in range(h_q):
                    g = h // (h_q // h_kv)
                    s = scale * (K[:vis, g] @ f64(q[q0 + i, h]))
                    p = np.exp(s - s.max())
                    p /= p.sum()
                    out[q0 + i, h] = p @ V[:vis, g]
        return out
    return fn


def _mutant_slots(kind):
    def fn(bt, start, end, bsz):
        if kind == "offset_from_start":
            return [bt[p // bsz] * bsz + (p - start) % bsz for p in range(start, end)]
        if kind == "table_by_offset":
            return [bt[(p % bsz) % len(bt)] * bsz + p // bsz for p in range(start, end)]
        return [bt[p // bsz] + p % bsz for p in range(start, end)]  # "no_block_scale"
    return fn


@pytest.mark.parametrize("kind", ["drop_last_token", "logical_block_as_physical", "gqa_modulo",
                                  "no_scale", "unnormalised", "k_for_v"])
def test_pins_catch_planted_decode_mistake(kind):
    mutant = _mutant_decode(kind)
    checks = [check_decode_vs_sdpa, check_decode_permutation_invariance,
              check_single_token_is_value, check_equal_keys_give_mean_value]
    caught = 0
    for chk in checks:
        try:
            chk(mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


@pytest.mark.parametrize("kind", ["top_left_causal", "strict_causal"])
def test_pins_catch_planted_prefill_mistake(kind):
    with pytest.raises(AssertionError):
        check_prefill_vs_full_recompute(_mutant_prefill(kind))


@pytest.mark.parametrize("kind", ["offset_from_start", "table_by_offset", "no_block_scale"])
def test_pins_catch_planted_slot_mistake(kind):
    with pytest.raises(AssertionError):
        check_range_examples(_mutant_slots(kind))


def test_unmutated_checks_pass():
    check_decode_vs_sdpa(_mutant_decode("none"))
    check_prefill_vs_full_recompute(_mutant_prefill("none"))
