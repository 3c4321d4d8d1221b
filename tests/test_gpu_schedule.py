"""End to end over the path, following the prefill scheduling example of
"12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.9 Scheduler: prompts
A (512 tokens), B (200) and C (3000) with a budget of 1,024 tokens per step
and 256-token blocks. Step 1 prefills A and B in one varlen batch; C is a
chunked prefill of 1024 / 1024 / 952 tokens over three steps; then A, B and
C decode one token together.

Every step goes through the native block manager (tables), the metadata
builder (slots, cu_seqlens), pa_store_kv and the attention entry points.
The chunked outputs must equal the fp64 oracle's one-shot prefill of each
whole prompt, and the caches must equal the oracle store of every step."""

import numpy as np
import pytest

import oracle
from gpu_helpers import NAN_BF16, assert_close, dev_bf16, dev_i32, host_bits, host_f64
from oracle.block_manager import Seq
from paged_kv_cache_kvcache_amd import binding as B
from paged_kv_cache_kvcache_amd import workloads as W
from paged_kv_cache_kvcache_amd.block_manager import BlockManager

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H_Q, H_KV, D, BS = 32, 8, 128, 256
PROMPTS = {"A": 512, "B": 200, "C": 3000}
STEPS = [[("A", 0, 512), ("B", 0, 200)],
         [("C", 0, 1024)],
         [("C", 1024, 2048)],
         [("C", 2048, 3000)]]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def test_scheduler_example_chunked_prefill_then_decode():
    rng = np.random.default_rng(91)
    num_blocks = 24
    bm = BlockManager(num_blocks, BS)
    seqs = {n: Seq(rng.integers(0, 150000, size=L).tolist(), BS) for n, L in PROMPTS.items()}
    total = {n: L + 1 for n, L in PROMPTS.items()}  # the decode step adds one token
    qs = {n: W.normal_bf16(rng, (total[n], H_Q, D)) for n in PROMPTS}
    ks = {n: W.normal_bf16(rng, (total[n], H_KV, D)) for n in PROMPTS}
    vs = {n: W.normal_bf16(rng, (total[n], H_KV, D)) for n in PROMPTS}
    kc_ref = np.full((num_blocks, BS, H_KV, D), NAN_BF16, dtype=np.uint16)
    vc_ref = kc_ref.copy()
    kc, vc = dev_bf16(kc_ref), dev_bf16(vc_ref)
    scale = 1.0 / np.sqrt(D)
    got = {n: np.full((L, H_Q, D), np.nan) for n, L in PROMPTS.items()}

    for i, step in enumerate(STEPS):
        names = [n for n, _, _ in step]
        for n in names:
            if not seqs[n].block_table:
                hits = bm.can_allocate(seqs[n])
                assert hits == 0  # random prompts share no block
                bm.allocate(seqs[n], hits)
        starts = np.array([s for _, s, _ in step], dtype=np.int32)
        ends = np.array([e for _, _, e in step], dtype=np.int32)
        assert all(seqs[n].num_cached_tokens == s for n, s, _ in step)
        tables = W.pad_tables([seqs[n].block_table for n in names])
        slots, cu_q, cu_k = B.pa_build_metadata(tables, starts, ends, BS)
        k_new = np.concatenate([ks[n][s:e] for n, s, e in step])
        v_new = np.concatenate([vs[n][s:e] for n, s, e in step])
        q = np.concatenate([qs[n][s:e] for n, s, e in step])
        print("step %d: %s, %d new tokens" % (i + 1, names, len(q)), flush=True)
        B.pa_store_kv(dev_bf16(k_new), dev_bf16(v_new), kc, vc, dev_i32(slots))
        kc_ref, vc_ref = oracle.store_kv(kc_ref, vc_ref, k_new, v_new, slots)
        qd = dev_bf16(q)
        out = torch.empty_like(qd)
        B.pa_prefill_varlen(qd, kc, vc, dev_i32(cu_q), dev_i32(cu_k), int((ends - starts).max()),
                            int(ends.max()), dev_i32(tables), scale, out)
        torch.cuda.synchronize()
        o = host_f64(out)
        for j, (n, s, e) in enumerate(step):
            got[n][s:e] = o[cu_q[j]:cu_q[j + 1]]
            bm.hash_blocks(seqs[n], e - s)
            seqs[n].num_cached_tokens += e - s
    assert np.array_equal(host_bits(kc), kc_ref) and np.array_equal(host_bits(vc), vc_ref)
    assert seqs["C"].num_cached_tokens == 3000 and len(seqs["C"].block_table) == 12

    # chunked prefill == one-shot prefill of the whole prompt (every row)
    for n, L in PROMPTS.items():
        ref = oracle.prefill_one(qs[n][:L], kc_ref, vc_ref, seqs[n].block_table, L, scale)
        mx, mean = assert_close(got[n][:L], ref, "chunked prefill %s" % n)
        print("  %s: max abs %.3g mean abs %.3g" % (n, mx, mean), flush=True)

    # step 5: A, B and C decode one token together (A spills into a new block)
    names = list(PROMPTS)
    for n in names:
        seqs[n].token_ids.append(int(rng.integers(0, 150000)))
        assert bm.can_append(seqs[n])
        bm.may_append(seqs[n])
    assert len(seqs["A"].block_table) == 3 and len(seqs["B"].block_table) == 1
    ctx = np.array([total[n] for n in names], dtype=np.int32)
    tables = W.pad_tables([seqs[n].block_table for n in names])
    slots, _, _ = B.pa_build_metadata(tables, ctx - 1, ctx, BS)
    k_new = np.stack([ks[n][-1] for n in names])
    v_new = np.stack([vs[n][-1] for n in names])
    q = np.stack([qs[n][-1] for n in names])
    B.pa_store_kv(dev_bf16(k_new), dev_bf16(v_new), kc, vc, dev_i32(slots))
    kc_ref, vc_ref = oracle.store_kv(kc_ref, vc_ref, k_new, v_new, slots)
    qd = dev_bf16(q)
    out = torch.empty_like(qd)
    B.pa_decode(qd, kc, vc, dev_i32(tables), dev_i32(ctx), scale, out,
                max_context_len=int(ctx.max()))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc), kc_ref) and np.array_equal(host_bits(vc), vc_ref)
    ref = oracle.decode(q, kc_ref, vc_ref, tables, ctx, scale)
    mx, mean = assert_close(host_f64(out), ref, "decode after chunked prefill")
    print("  decode: max abs %.3g mean abs %.3g" % (mx, mean), flush=True)
