"""GPU parity of the fused decode step (pa_decode_step: store of each
sequence's newest token + paged decode in one pass), and of that step
captured in a HIP graph and replayed with new inputs, against the fp64
oracle (store bit-exact; attention max-abs 1e-2 / mean-abs 1e-3)."""

import numpy as np
import pytest

import oracle
from gpu_helpers import (assert_close, check_whole_output, dev_bf16, dev_i32, host_bits, host_f64,
                         poison_unused)
from paged_kv_cache_kvcache_amd import binding as B
from paged_kv_cache_kvcache_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def step_slots(case):
    slots, _, _ = B.pa_build_metadata(case.block_tables, case.starts, case.context_lens, 256)
    full = np.full(case.batch, -1, dtype=np.int32)
    full[case.context_lens > 0] = slots
    return full


def check_step(case, out_f64, caches, before, slots, rows=None):
    kref, vref = oracle.store_kv(before[0], before[1], case.k_new, case.v_new, slots)
    assert np.array_equal(host_bits(caches[0]), kref) and np.array_equal(host_bits(caches[1]), vref)
    ref = oracle.decode(case.q, kref, vref, case.block_tables, case.context_lens, case.scale,
                        rows=rows)
    sel = slice(None) if rows is None else list(rows)
    return assert_close(out_f64[sel], ref[sel], case.name)


@pytest.mark.parametrize("name", ["tiny", "qwen3-0.6b"])
def test_fused_step_full_oracle(name):
    case = W.make_case(name)
    print("fused step:", name, flush=True)
    slots = step_slots(case)
    kc0, vc0 = poison_unused(case.k_cache, case.v_cache, case.block_tables, case.starts, 256)
    kc, vc = dev_bf16(kc0), dev_bf16(vc0)
    q = dev_bf16(case.q)
    out = torch.empty_like(q)
    B.pa_decode_step(q, dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots),
                     dev_i32(case.block_tables), dev_i32(case.context_lens), case.scale, out,
                     max_context_len=int(case.context_lens.max()))
    torch.cuda.synchronize()
    check_step(case, host_f64(out), (kc, vc), (kc0, vc0), slots)


@pytest.mark.parametrize("name", ["qwen3-8b", "gqa8"])
def test_fused_step_full_size_and_matches_unfused(name):
    case = W.make_case(name)
    print("fused step: %s" % name, flush=True)
    slots = step_slots(case)
    kc, vc = dev_bf16(case.k_cache), dev_bf16(case.v_cache)
    q, k_new, v_new = dev_bf16(case.q), dev_bf16(case.k_new), dev_bf16(case.v_new)
    bt, ctx, sl = dev_i32(case.block_tables), dev_i32(case.context_lens), dev_i32(slots)
    max_ctx = int(case.context_lens.max())
    out_f = torch.empty_like(q)
    B.pa_decode_step(q, k_new, v_new, kc, vc, sl, bt, ctx, case.scale, out_f,
                     max_context_len=max_ctx)
    # the unfused pair on the caches the fused step left behind (its store
    # rewrites the same rows with the same values)
    out_u = torch.empty_like(q)
    B.pa_store_kv(k_new, v_new, kc, vc, sl)
    B.pa_decode(q, kc, vc, bt, ctx, case.scale, out_u, max_context_len=max_ctx)
    torch.cuda.synchronize()
    kref, vref = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    assert np.array_equal(host_bits(kc), kref) and np.array_equal(host_bits(vc), vref)
    del kref, vref
    check_whole_output("decode", name, out_f)
    d = np.abs(host_f64(out_f) - host_f64(out_u))
    assert d.max() <= 1e-2 and d.mean() <= 1e-4, (d.max(), d.mean())


def test_fused_step_padding_rows_and_strided_new_tokens():
    lens = [0, 1, 255, 256, 257, 0, 1500]
    case = W.decode_case(32, 8, 128, lens, seed=121)
    slots = step_slots(case)
    kc0, vc0 = poison_unused(case.k_cache, case.v_cache, case.block_tables, case.starts, 256)
    kc, vc = dev_bf16(kc0), dev_bf16(vc0)
    qkv = torch.empty(len(lens), 48, 128, dtype=torch.bfloat16, device="cuda")
    qkv[:, :32] = dev_bf16(case.q)
    qkv[:, 32:40] = dev_bf16(case.k_new)
    qkv[:, 40:] = dev_bf16(case.v_new)
    q = qkv[:, :32].contiguous()
    out = torch.empty_like(q)
    B.pa_decode_step(q, qkv[:, 32:40], qkv[:, 40:], kc, vc, dev_i32(slots),
                     dev_i32(case.block_tables), dev_i32(case.context_lens), case.scale, out,
                     max_context_len=max(lens))
    torch.cuda.synchronize()
    o = host_f64(out)
    check_step(case, o, (kc, vc), (kc0, vc0), slots)
    assert np.all(o[[0, 5]] == 0)


@pytest.mark.parametrize("h_q", [32, 64])
def test_graph_replay_of_the_step_with_new_inputs(h_q):
    """The per-layer decode step captured once in a graph (static input
    buffers, padding rows with slot -1 / length 0, as a graph bucket would
    have), then replayed three times with new q, new tokens and longer
    contexts copied into the static buffers, with eager work between the
    replays. Every replay must equal the oracle and the eager step. 64
    q-heads per 8 kv-heads runs the matrix-core kernel (LDS staging)."""
    rng = np.random.default_rng(122)
    h_kv, d, bsz = 8, 128, 8
    base = [300, 1, 4000, 256, 700]  # 5 live rows, 3 padding rows
    max_blocks = 20
    nb = 128
    kc_h = W.normal_bf16(rng, (nb, 256, h_kv, d))
    vc_h = W.normal_bf16(rng, (nb, 256, h_kv, d))
    tables = np.full((bsz, max_blocks), -1, dtype=np.int32)
    perm = rng.permutation(nb)
    for b in range(len(base)):
        tables[b, :max_blocks] = perm[b * max_blocks:(b + 1) * max_blocks]
    kc, vc = dev_bf16(kc_h), dev_bf16(vc_h)
    s_q = torch.zeros(bsz, h_q, d, dtype=torch.bfloat16, device="cuda")
    s_k = torch.zeros(bsz, h_kv, d, dtype=torch.bfloat16, device="cuda")
    s_v = torch.zeros(bsz, h_kv, d, dtype=torch.bfloat16, device="cuda")
    s_slots = torch.full((bsz,), -1, dtype=torch.int32, device="cuda")
    s_ctx = torch.zeros(bsz, dtype=torch.int32, device="cuda")
    s_bt = dev_i32(tables)
    s_out = torch.empty_like(s_q)
    max_ctx = max_blocks * 256
    ws = torch.zeros(B.pa_decode_workspace_size(h_q, kc, bsz, max_ctx), dtype=torch.uint8,
                     device="cuda")

    def step():
        B.pa_decode_step(s_q, s_k, s_v, kc, vc, s_slots, s_bt, s_ctx, 1 / np.sqrt(d), s_out,
                         max_context_len=max_ctx, workspace=ws)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    cache_k, cache_v = kc_h.copy(), vc_h.copy()
    for it in range(3):
        lens = np.zeros(bsz, dtype=np.int32)
        lens[:len(base)] = [x + it for x in base]
        qn = W.normal_bf16(rng, (bsz, h_q, d))
        kn = W.normal_bf16(rng, (bsz, h_kv, d))
        vn = W.normal_bf16(rng, (bsz, h_kv, d))
        slots = np.full(bsz, -1, dtype=np.int32)
        live = lens > 0
        starts = np.maximum(lens - 1, 0)
        slots[live] = B.pa_build_metadata(tables[live], starts[live], lens[live], 256)[0]
        s_q.copy_(dev_bf16(qn))
        s_k.copy_(dev_bf16(kn))
        s_v.copy_(dev_bf16(vn))
        s_slots.copy_(dev_i32(slots))
        s_ctx.copy_(dev_i32(lens))
        g.replay()
        torch.cuda.synchronize()
        got = host_f64(s_out)
        # eager work between replays, then the eager step on a copy
        kc_e, vc_e = kc.clone(), vc.clone()
        out_e = torch.empty_like(s_q)
        B.pa_decode_step(s_q, s_k, s_v, kc_e, vc_e, s_slots, s_bt, s_ctx, 1 / np.sqrt(d), out_e,
                         max_context_len=max_ctx)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out_e), host_bits(s_out)), "replay %d != eager" % it
        cache_k, cache_v = oracle.store_kv(cache_k, cache_v, kn, vn, slots)
        assert np.array_equal(host_bits(kc), cache_k) and np.array_equal(host_bits(vc), cache_v)
        ref = oracle.decode(qn, cache_k, cache_v, tables, lens, 1 / np.sqrt(d))
        assert_close(got, ref, "replay %d" % it)
        assert np.all(got[~live] == 0)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_of_several_layers_shares_one_workspace(fused):
    """Four layers, each with its own pool, captured as one graph (the
    shape of a model's decode step: the layers' decode calls share one
    workspace, whose arrival counters each call leaves at zero for the
    next), replayed three times with new q and new tokens and eager work
    between the replays. Every layer's output of every replay equals the
    eager step's bit for bit, and the oracle's; the caches hold every
    stored token. Lengths vary so that long sequences are split over
    grabs and merged."""
    rng = np.random.default_rng(321)
    h_q, h_kv, d, layers = 32, 8, 128, 4
    lens = np.array([3000, 1, 0, 777, 4096, 256, 2500, 90], dtype=np.int32)
    bsz = len(lens)
    max_blocks = 16
    nb = bsz * max_blocks + 4
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((bsz, max_blocks), -1, dtype=np.int32)
    for b in range(bsz):
        tables[b] = perm[b * max_blocks:(b + 1) * max_blocks]
    host = [(W.normal_bf16(rng, (nb, 256, h_kv, d)), W.normal_bf16(rng, (nb, 256, h_kv, d)))
            for _ in range(layers)]
    caches = [(dev_bf16(k), dev_bf16(v)) for k, v in host]
    s_q = torch.zeros(bsz, h_q, d, dtype=torch.bfloat16, device="cuda")
    s_k = torch.zeros(bsz, h_kv, d, dtype=torch.bfloat16, device="cuda")
    s_v = torch.zeros(bsz, h_kv, d, dtype=torch.bfloat16, device="cuda")
    live = lens > 0
    slots = np.full(bsz, -1, dtype=np.int32)
    slots[live] = B.pa_build_metadata(tables[live], np.maximum(lens - 1, 0)[live], lens[live],
                                      256)[0]
    s_slots, s_bt, s_ctx = dev_i32(slots), dev_i32(tables), dev_i32(lens)
    outs = [torch.empty_like(s_q) for _ in range(layers)]
    max_ctx = max_blocks * 256
    ws = torch.zeros(B.pa_decode_workspace_size(h_q, caches[0][0], bsz, max_ctx),
                     dtype=torch.uint8, device="cuda")
    scale = 1 / np.sqrt(d)

    def step(cs, os_):
        for (kc, vc), out in zip(cs, os_):
            if fused:
                B.pa_decode_step(s_q, s_k, s_v, kc, vc, s_slots, s_bt, s_ctx, scale, out,
                                 max_context_len=max_ctx, workspace=ws)
            else:
                B.pa_store_kv(s_k, s_v, kc, vc, s_slots)
                B.pa_decode(s_q, kc, vc, s_bt, s_ctx, scale, out, max_context_len=max_ctx,
                            workspace=ws)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(caches, outs)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(caches, outs)
    torch.cuda.synchronize()

    ref_caches = [(k.copy(), v.copy()) for k, v in host]
    for it in range(3):
        qn = W.normal_bf16(rng, (bsz, h_q, d))
        kn = W.normal_bf16(rng, (bsz, h_kv, d))
        vn = W.normal_bf16(rng, (bsz, h_kv, d))
        s_q.copy_(dev_bf16(qn))
        s_k.copy_(dev_bf16(kn))
        s_v.copy_(dev_bf16(vn))
        g.replay()
        torch.cuda.synchronize()
        got = [host_bits(o) for o in outs]
        # eager work between replays: the same step on copies of the caches
        eager_caches = [(kc.clone(), vc.clone()) for kc, vc in caches]
        eager_outs = [torch.empty_like(s_q) for _ in range(layers)]
        step(eager_caches, eager_outs)
        torch.cuda.synchronize()
        for l in range(layers):
            assert np.array_equal(host_bits(eager_outs[l]), got[l]), \
                "replay %d layer %d != eager" % (it, l)
            ref_caches[l] = oracle.store_kv(ref_caches[l][0], ref_caches[l][1], kn, vn, slots)
            assert np.array_equal(host_bits(caches[l][0]), ref_caches[l][0])
            assert np.array_equal(host_bits(caches[l][1]), ref_caches[l][1])
        for l in (0, layers - 1):
            ref = oracle.decode(qn, ref_caches[l][0], ref_caches[l][1], tables, lens, scale)
            assert_close(host_f64(outs[l]), ref, "replay %d layer %d" % (it, l))
            assert np.all(host_f64(outs[l])[~live] == 0)
