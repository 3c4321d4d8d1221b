#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

A step is one pass of the decode hot path over the Qwen3-8B-shaped batch
(32 q / 8 kv heads, head_dim 128, block 256, 256 sequences with context
U[512, 8192]): ``pa_store_kv`` of the 256 new tokens, then ``pa_decode``.
Inputs are seeded synthetic data already resident in HBM when timing starts.

Prints ONE JSON line: the metric (KV GB/s of the step's algorithmic bytes,
with % of HBM peak and tokens/s beside it), the roofline of the dominant
call (pa_decode) timed with HIP events on its stream, and the CPU oracle
baseline on a bounded sample. A default run adds, under "configs", the
other workloads with their own rooflines and CPU baselines: the
Qwen3-0.6B-shaped decode (64 sequences, U[128, 4096]), the long-context
decode (32 x 16,384) and the prefix-cached prefill (bf16 MFMA roofline)
with its 18,342-token store (HBM roofline). ``--only`` times the headline
workload alone and ``--prefill-only`` the prefill workload alone (for
profiling one workload).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0
LAYERS_QWEN3_8B = 36
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_decode_qwen3-8b.json")


def pmc_decode_file(config: str) -> str:
    """The committed counter record of a decode workload (may not exist)."""
    return os.path.join(ROOT, "profiles", "pmc_decode_%s.json" % config)
PMC_PREFILL_FILE = os.path.join(ROOT, "profiles", "pmc_prefill_prefix1024.json")
PMC_STORE_FILE = os.path.join(ROOT, "profiles", "pmc_store_prefill18k.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_kvcache_amd", "csrc", "decode.hip")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_kvcache_amd", "csrc", "prefill.hip")
STORE_SRC = os.path.join(ROOT, "paged_kv_cache_kvcache_amd", "csrc", "store_kv.hip")


def decode_bytes(case) -> int:
    """Algorithmic HBM bytes of one pa_decode call: every K and V row of every
    context token once (2 * H_kv * d * 2 bytes per token), q read and out
    written once, one table entry per block and one length per sequence."""
    import numpy as np
    ctx = case.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2 * case.batch * case.num_q_heads * case.head_dim * 2
    tables = int((-(-ctx // case.block_size)).sum()) * 4
    return kv + qo + tables + 4 * case.batch


def store_bytes(n_tokens: int, h_kv: int, d: int) -> int:
    """K and V rows read once and written once, plus one slot per token."""
    return 2 * 2 * n_tokens * h_kv * d * 2 + 4 * n_tokens


def prefill_flops(starts, ends, h_q: int, d: int) -> float:
    """Causal-exact FLOPs: query at position p attends p+1 keys; QK^T and PV
    each cost 2*d FLOPs per (query, key, head)."""
    total = 0
    for s, e in zip(starts, ends):
        s, e = int(s), int(e)
        total += (e * (e + 1) - s * (s + 1)) // 2  # sum over p in [s, e) of (p + 1)
    return float(total) * h_q * 4 * d


def src_hash(path: str) -> str:
    """Digest of a kernel source's code: `//` comments and blank space are
    left out, so a comment edit does not retire counters taken on the same
    code."""
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    code = "\n".join(" ".join(re.sub(r"//.*", "", line).split()) for line in text.splitlines())
    code = re.sub(r"\n+", "\n", code).strip()
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile(pmc_file: str, kernel_src: str, mode: str | None,
                         block_size: int = 256, config: str | None = None):
    """HBM bytes per launch of a call from a committed rocprofv3 counter
    summary, or None if it is missing, was taken for another workload, step
    mode or block size, or on a different kernel source."""
    try:
        with open(pmc_file) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("source_sha256_16") != src_hash(kernel_src) or rec.get("step_mode") != mode
            or rec.get("block_size") != block_size or rec.get("config") != config):
        return None
    return rec.get("traffic_bytes_per_launch")


def _oracle_rows(rows):
    """Worker: the oracle's decode of the given sequences of the inherited case."""
    import oracle
    c = _CPU_CASE
    for b in rows:
        oracle.decode_one(c.q[b], c.k_cache, c.v_cache, c.block_tables[b], int(c.context_lens[b]),
                          c.scale)
    return len(rows)


def _oracle_prefill_piece(task):
    """Worker: the oracle's prefill of query rows [lo, hi) of sequence b."""
    import oracle
    b, lo, hi = task
    c, cu_q = _CPU_CASE, _CPU_CU_Q
    q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
    oracle.prefill_one(c.q[q0:q1], c.k_cache, c.v_cache, c.block_tables[b], int(c.ends[b]),
                       c.scale, query_rows=range(lo, hi))
    return task


_CPU_CASE = None
_CPU_CU_Q = None


def cpu_baseline_child(args) -> int:
    """Runs in a fresh interpreter that never touches the GPU: draws the same
    workload and times the fp64 oracle on it in a pool of worker processes,
    one per host core (at most 16, one thread each), until the batch is done
    or about ``--cpu-budget`` seconds have passed. Decode: one sequence per
    task, in batch order. Prefill: pieces of 64 query rows, in batch order."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from paged_kv_cache_kvcache_amd import workloads as W
    global _CPU_CASE, _CPU_CU_Q
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    case = W.make_case(args.config, block_size=args.block_size, threads=cores)
    _CPU_CASE = case
    prefill = args.config == "prefill"
    if prefill:
        qlens = (case.ends - case.starts).astype(np.int64)
        _CPU_CU_Q = np.concatenate([[0], np.cumsum(qlens)])
        tasks = [(b, lo, min(int(qlens[b]), lo + 64)) for b in range(case.batch)
                 for lo in range(0, int(qlens[b]), 64)]
        fn = _oracle_prefill_piece
    else:
        tasks = [[b] for b in range(case.batch)]
        fn = _oracle_rows
    done = []
    with threadpool_limits(1):
        pool = mp.get_context("fork").Pool(cores)
        try:
            t0 = time.perf_counter()
            for r in pool.imap(fn, tasks):
                done.append(r)
                if time.perf_counter() - t0 >= args.cpu_budget:
                    break
            el = time.perf_counter() - t0
        finally:
            pool.terminate()
    if prefill:
        # causal-exact FLOPs of the rows done: query row i of sequence b sits
        # at position starts[b] + i and sees that many keys plus one
        flops = 0.0
        rows = 0
        for b, lo, hi in done:
            s0 = int(case.starts[b])
            flops += prefill_flops([s0 + lo], [s0 + hi], case.num_q_heads, case.head_dim)
            rows += hi - lo
        total_rows = int((case.ends - case.starts).sum())
        print(json.dumps({
            "value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "fp64 numpy oracle prefill of %d of %d query rows (%d pieces of up to 64 "
                      "rows, batch order) in %d worker processes of one thread each, %.2f s; "
                      "store not included" % (rows, total_rows, len(done), cores, el),
            "q_tokens_per_s": round(rows / el, 3)}), flush=True)
        return 0
    n_seqs = sum(len(r_) for r_ in tasks[:len(done)])
    tokens = int(case.context_lens[:n_seqs].sum())
    kv = tokens * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2 * n_seqs * case.num_q_heads * case.head_dim * 2
    print(json.dumps({
        "value": round((kv + qo) / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": "fp64 numpy oracle decode of the first %d of %d sequences (%d context tokens) "
                  "in %d worker processes of one thread each, %.2f s; store not included" % (
                      n_seqs, case.batch, tokens, cores, el),
        "tokens_per_s_per_layer": round(n_seqs / el, 3)}), flush=True)
    return 0


def cpu_baseline(args, config: str):
    """The CPU oracle baseline of one workload, measured in a child process
    (see cpu_baseline_child) so that its workers fork from a process without
    a GPU context."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child",
           "--block-size", str(args.block_size), "--cpu-budget", str(args.cpu_budget)]
    cmd += ["--prefill-only"] if config == "prefill" else ["--config", config]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=args.cpu_budget + 600)
    if r.returncode != 0:
        raise RuntimeError("CPU baseline failed (%d): %s" % (r.returncode, r.stderr[-2000:]))
    return json.loads(r.stdout.strip().splitlines()[-1])


def _dev(torch, dev):
    import numpy as np

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf(a):
        return t(a.view(np.int16)).view(torch.bfloat16)
    return t, bf


def run_prefill(args, torch, B, W, dev, warmup=None, warm_s=0.0):
    """The prefix-cached prefill workload: pa_store_kv of the 18,342 new
    tokens, then pa_prefill_varlen. Two rooflines: the prefill kernel
    (causal-exact FLOPs, dense bf16 MFMA peak) and the store (bytes, HBM)."""
    case = W.make_case("prefill")
    slots, cu_q, cu_k = B.pa_build_metadata(case.block_tables, case.starts, case.ends,
                                            case.block_size)
    t, bf = _dev(torch, dev)
    kc, vc = bf(case.k_cache), bf(case.v_cache)
    k_new, v_new, q = bf(case.k_new), bf(case.v_new), bf(case.q)
    out = torch.empty_like(q)
    slots_d, cuq_d, cuk_d, bt_d = t(slots), t(cu_q), t(cu_k), t(case.block_tables)
    qlens = case.ends - case.starts
    mq, mk = int(qlens.max()), int(case.ends.max())

    def store():
        B.pa_store_kv(k_new, v_new, kc, vc, slots_d)

    def attn():
        B.pa_prefill_varlen(q, kc, vc, cuq_d, cuk_d, mq, mk, bt_d, case.scale, out)

    def both():
        store()
        attn()

    warm(torch, dev, both, max(1, args.warmup if warmup is None else warmup), warm_s)
    n = max(3, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        store()
        ev[i][1].record()
        attn()
        ev[i][2].record()
    torch.cuda.synchronize(dev)
    t_store = sum(e[0].elapsed_time(e[1]) for e in ev) / n * 1e-3
    t_attn = sum(e[1].elapsed_time(e[2]) for e in ev) / n * 1e-3
    flops = prefill_flops(case.starts, case.ends, case.num_q_heads, case.head_dim)
    n_q = int(qlens.sum())
    sb = store_bytes(n_q, case.num_kv_heads, case.head_dim)
    tflops = flops / t_attn / 1e12
    store_gbs = sb / t_store / 1e9
    return {
        "workload": W.DESCRIPTIONS["prefill"] + "; step = store of the %d new tokens + prefill"
                    % n_q,
        "metric": "varlen causal prefill over paged K/V: TFLOP/s (causal-exact) and query "
                  "tokens/s",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "q_tokens": n_q,
        "ms_per_call": {"pa_store_kv": round(t_store * 1e3, 5),
                        "pa_prefill_varlen": round(t_attn * 1e3, 5)},
        "q_tokens_per_s": round(n_q / (t_store + t_attn), 1),
        "algorithmic": {"prefill_flops": flops, "store_bytes": sb},
        "roofline": {"bound": "mfma", "kernel": "pa_prefill_varlen (prefill32_kernel)",
                     "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile(PMC_PREFILL_FILE, PREFILL_SRC, None)},
        "store": {"tokens": n_q, "value": round(store_gbs, 1), "unit": "GB/s",
                  "roofline": {"bound": "hbm", "kernel": "pa_store_kv (store_kv_vec16_kernel)",
                               "achieved": round(store_gbs, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(store_gbs / HBM_PEAK_GBS, 4),
                               "traffic": traffic_from_profile(PMC_STORE_FILE, STORE_SRC,
                                                               None)}},
    }


def run_mixed(args, torch, B, W, dev):
    """A mixed step (decode rows + chunked-prefill rows) in one varlen launch."""
    import numpy as np
    case = W.make_case("mixed")
    slots, cu_q, cu_k = B.pa_build_metadata(case.block_tables, case.starts, case.ends,
                                            case.block_size)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf(a):
        return t(a.view(np.int16)).view(torch.bfloat16)

    kc, vc = bf(case.k_cache), bf(case.v_cache)
    k_new, v_new, q = bf(case.k_new), bf(case.v_new), bf(case.q)
    out = torch.empty_like(q)
    slots_d, cuq_d, cuk_d, bt_d = t(slots), t(cu_q), t(cu_k), t(case.block_tables)
    qlens = case.ends - case.starts
    mq, mk = int(qlens.max()), int(case.ends.max())

    n_dec = case.meta["decode_rows"]
    ws = torch.zeros(max(16, B.load().pa_mixed_workspace_size(
        B.ctypes.byref(B._desc_from_cache(kc, case.num_q_heads)), n_dec, mk)),
        dtype=torch.uint8, device=dev)

    def step_mixed():
        B.pa_store_kv(k_new, v_new, kc, vc, slots_d)
        B.pa_mixed_varlen(q, kc, vc, cuq_d, cuk_d, n_dec, mq, mk, bt_d, case.scale, out,
                          workspace=ws)

    def step_prefill_only():
        B.pa_store_kv(k_new, v_new, kc, vc, slots_d)
        B.pa_prefill_varlen(q, kc, vc, cuq_d, cuk_d, mq, mk, bt_d, case.scale, out)

    def timed(step):
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize(dev)
        n = max(3, args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / n

    ms = timed(step_mixed)
    ms_single = timed(step_prefill_only)
    kv = int(case.ends.astype(np.int64).sum()) * case.num_kv_heads * case.head_dim * 4
    return {"workload": W.DESCRIPTIONS["mixed"], "q_tokens": int(qlens.sum()),
            "entry": "pa_store_kv + pa_mixed_varlen",
            "ms_per_step": round(ms, 4), "kv_GBps": round(kv / (ms * 1e-3) / 1e9, 1),
            "q_tokens_per_s": round(int(qlens.sum()) / (ms * 1e-3), 1),
            "ms_per_step_single_prefill_launch": round(ms_single, 4)}


def run_decode(args, torch, B, W, dev, config: str, mode: str = "separate",
               graph: bool = False, replicas: int = 0, warmup=None, warm_s=0.0) -> dict:
    """One decode workload: W untimed steps, then K steps back to back
    between two events (the step time), with an event after each call inside
    that region (per-call times; the roofline's). A step is
    pa_store_kv of the batch's new tokens + pa_decode (mode "separate") or
    pa_decode_step (mode "fused"), optionally replayed as a HIP graph."""
    case = W.make_case(config, block_size=args.block_size)
    t, bf = _dev(torch, dev)
    slots, _, _ = B.pa_build_metadata(case.block_tables, case.starts, case.context_lens,
                                      case.block_size)
    kc, vc = bf(case.k_cache), bf(case.v_cache)
    q, k_new, v_new = bf(case.q), bf(case.k_new), bf(case.v_new)
    out = torch.empty_like(q)
    slots_d, bt_d, ctx_d = t(slots), t(case.block_tables), t(case.context_lens)
    max_ctx = int(case.context_lens.max())
    ws_bytes = B.pa_decode_workspace_size(case.num_q_heads, kc, case.batch, max_ctx)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # A batch whose K/V are within a small multiple of the 256 MB last-level
    # cache (MALL) could be partly served from it on back-to-back steps;
    # consecutive steps then read different copies of the pool (2.1 GB at
    # 32 x 16,384 tokens: two copies measured 0.3% slower than one).
    kv_bytes = decode_bytes(case)
    replicas = 1 if graph else (replicas or (1 if kv_bytes >= (4 << 30) else 2))
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(replicas - 1)]
    turn = [0]

    def store(pool):
        B.pa_store_kv(k_new, v_new, pool[0], pool[1], slots_d)

    def decode(pool):
        B.pa_decode(q, pool[0], pool[1], bt_d, ctx_d, case.scale, out, max_context_len=max_ctx,
                    workspace=ws)

    def fused(pool):
        B.pa_decode_step(q, k_new, v_new, pool[0], pool[1], slots_d, bt_d, ctx_d, case.scale, out,
                         max_context_len=max_ctx, workspace=ws)

    if mode == "fused":
        calls = [("pa_decode_step", fused)]
    else:
        calls = [("pa_store_kv", store), ("pa_decode", decode)]

    def next_pool():
        pool = pools[turn[0] % len(pools)]
        turn[0] += 1
        return pool

    def step():
        pool = next_pool()
        for _, fn in calls:
            fn(pool)

    if warmup is None:
        warmup = args.warmup
    warm(torch, dev, step, warmup, warm_s)
    run = step
    if graph:
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize(dev)
        run = g.replay
        for _ in range(warmup):
            run()
        torch.cuda.synchronize(dev)

    # K steps back to back, timed between two events; inside that region an
    # event after each call gives the per-call durations (the roofline's).
    # A replayed graph has no per-call events: its calls are timed in a
    # second pass of eager steps.
    n = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(n)]
    torch.cuda.synchronize(dev)
    start.record()
    for i in range(n):
        if graph:
            run()
            continue
        pool = next_pool()
        ev[i][0].record()
        for j, (_, fn) in enumerate(calls):
            fn(pool)
            ev[i][j + 1].record()
    end.record()
    torch.cuda.synchronize(dev)
    ms_step = start.elapsed_time(end) / n
    if graph:
        for i in range(n):
            pool = next_pool()
            ev[i][0].record()
            for j, (_, fn) in enumerate(calls):
                fn(pool)
                ev[i][j + 1].record()
        torch.cuda.synchronize(dev)
    ms_call = {name: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / n
               for j, (name, _) in enumerate(calls)}

    db = decode_bytes(case)
    sb = store_bytes(case.batch, case.num_kv_heads, case.head_dim)
    gbs = (db + sb) / (ms_step * 1e-3) / 1e9
    if mode == "fused":
        dom, dom_bytes = "pa_decode_step", db + sb
        dom_desc = "pa_decode_step (decode_stream_kernel: one launch, split-K over balanced " \
                   "grabs, merged in the kernel; the new tokens stored by it)"
    else:
        dom, dom_bytes = "pa_decode", db
        dom_desc = "pa_decode (decode_stream_kernel: one launch, split-K over balanced grabs, " \
                   "merged in the kernel)"
    dom_gbs = dom_bytes / (ms_call[dom] * 1e-3) / 1e9
    traffic = traffic_from_profile(pmc_decode_file(config), DECODE_SRC, mode, args.block_size,
                                   config)
    rec = {
        "workload": W.DESCRIPTIONS[config].replace("B 256", "B %d" % case.block_size)
                    + "; step = store of the batch's new tokens + decode, one layer",
        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms_step, 5),
        "global_batch": case.batch, "seq_len": max_ctx, "block_size": case.block_size,
        "pool_replicas": len(pools), "step_mode": mode + (" + hip graph" if graph else ""),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": {"per_layer": round(case.batch / (ms_step * 1e-3), 1)},
        "ms_per_call": {k: round(v, 5) for k, v in ms_call.items()},
        "algorithmic_bytes": {"decode": db, "store": sb},
        "roofline": {"bound": "hbm", "kernel": dom_desc,
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if config == "qwen3-8b":
        rec["tokens_per_s"]["model_36_layers_from_one_layer"] = round(
            case.batch / (LAYERS_QWEN3_8B * ms_step * 1e-3), 1)
    return rec


def run_model(args, torch, B, W, dev, layers: int = LAYERS_QWEN3_8B) -> dict:
    """A whole decode step of the attention of a Qwen3-8B-shaped model: per
    layer, the store of the batch's new tokens and decode over that layer's
    own KV pool (36 pools of the Qwen3-8B batch, ~5.2 GB each, so no layer
    is served from a cache filled by another), run four ways: eager or
    replayed as one HIP graph, with pa_store_kv + pa_decode (separate) or
    pa_decode_step (fused). The pools hold copies of one seeded pool (made
    on the device); q and the new tokens are shared by the layers."""
    case = W.make_case("qwen3-8b")
    t, bf = _dev(torch, dev)
    slots, _, _ = B.pa_build_metadata(case.block_tables, case.starts, case.context_lens,
                                      case.block_size)
    kc0, vc0 = bf(case.k_cache), bf(case.v_cache)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(layers - 1)]
    q, k_new, v_new = bf(case.q), bf(case.k_new), bf(case.v_new)
    out = torch.empty_like(q)
    slots_d, bt_d, ctx_d = t(slots), t(case.block_tables), t(case.context_lens)
    max_ctx = int(case.context_lens.max())
    ws = torch.zeros(max(16, B.pa_decode_workspace_size(case.num_q_heads, kc0, case.batch,
                                                        max_ctx)), dtype=torch.uint8, device=dev)

    def separate():
        for kc, vc in pools:
            B.pa_store_kv(k_new, v_new, kc, vc, slots_d)
            B.pa_decode(q, kc, vc, bt_d, ctx_d, case.scale, out, max_context_len=max_ctx,
                        workspace=ws)

    def fused():
        for kc, vc in pools:
            B.pa_decode_step(q, k_new, v_new, kc, vc, slots_d, bt_d, ctx_d, case.scale, out,
                             max_context_len=max_ctx, workspace=ws)

    def timed(run):
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / args.steps

    def graphed(step):
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize(dev)
        return g

    ms = {"eager separate": timed(separate), "eager fused": timed(fused)}
    g_sep, g_fused = graphed(separate), graphed(fused)
    ms["graph separate"] = timed(g_sep.replay)
    ms["graph fused"] = timed(g_fused.replay)
    del g_sep, g_fused
    db = decode_bytes(case) + store_bytes(case.batch, case.num_kv_heads, case.head_dim)
    best = min(ms, key=ms.get)
    return {
        "workload": "%d layers x (%s); step = per layer, store of the batch's new tokens + "
                    "decode over that layer's pool" % (layers, W.DESCRIPTIONS["qwen3-8b"]),
        "layers": layers, "pool_gib_per_layer": round(2 * kc0.numel() * 2 / 2 ** 30, 2),
        "ms_per_step": {k: round(v, 4) for k, v in ms.items()},
        "tokens_per_s": {k: round(case.batch / (v * 1e-3), 1) for k, v in ms.items()},
        "kv_gb_per_s": {k: round(layers * db / (v * 1e-3) / 1e9, 1) for k, v in ms.items()},
        "best": best,
    }


# The other decode workloads and the prefill workload, timed by a default run
# beside the Qwen3-8B headline (each with its own roofline and CPU baseline).
EXTRA_DECODE = ("qwen3-0.6b", "long", "skewed")
# Before each extra workload of the default line (the headline step takes
# exactly --warmup): at least this many untimed calls, and untimed calls until
# this much wall time has passed. The GPU's clock ramps over the first ~40 ms
# of sustained work: prefill calls took 0.73, 0.61, 0.59 and then a steady
# 0.575 ms over the first 20-call groups of one run.
EXTRA_WARMUP = 10
EXTRA_WARMUP_S = 0.06


def warm(torch, dev, fn, calls: int, seconds: float = 0.0) -> None:
    """`calls` untimed calls of fn, then more in groups of 10 until `seconds`
    of wall time have passed since the first."""
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize(dev)
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize(dev)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3-8b",
                    choices=["qwen3-8b", "qwen3-0.6b", "long", "gqa8", "gqa16", "skewed"])
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work per CPU baseline (0 = skip)")
    ap.add_argument("--only", action="store_true",
                    help="time only --config (no other workloads): for profiling one workload")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill workload (its store and prefill): for profiling")
    ap.add_argument("--mixed", action="store_true",
                    help="also time a mixed decode + chunked-prefill varlen step")
    ap.add_argument("--mode", default="separate", choices=["fused", "separate"],
                    help="fused: pa_decode_step (store + decode in one pass); separate: "
                         "pa_store_kv then pa_decode")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step in a HIP graph and time its replays")
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of the KV pool read in turn by consecutive steps (0: 2 when "
                         "the batch's K/V are under 2 GiB, so the last-level cache cannot serve "
                         "a step from the previous one; 1 with --graph)")
    ap.add_argument("--block-size", type=int, default=256,
                    help="tokens per cache block (power of two, 16..1024); same lengths")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--model-only", action="store_true",
                    help="time only the 36-layer decode step (eager and graph, separate and "
                         "fused)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:
        if args.prefill_only:
            args.config = "prefill"
        return cpu_baseline_child(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; --gpus %d (WORLD_SIZE %d) is not supported: the "
              "library has no multi-GPU path" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_kvcache_amd import binding as B
    from paged_kv_cache_kvcache_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": n, "launches": max(1, args.steps)}))
        return 0

    B.load()

    def progress(msg):
        print("bench: " + msg, file=sys.stderr, flush=True)

    if args.model_only:
        print(json.dumps(run_model(args, torch, B, W, dev)), flush=True)
        return 0
    if args.prefill_only:
        rec = run_prefill(args, torch, B, W, dev)
        rec["cpu_baseline"] = cpu_baseline(args, "prefill") if args.cpu_budget > 0 else None
        print(json.dumps(rec), flush=True)
        return 0

    progress("%s decode" % args.config)
    head = run_decode(args, torch, B, W, dev, args.config, args.mode, args.graph, args.replicas)
    torch.cuda.empty_cache()
    rec = {
        "metric": "paged decode: KV GB/s (% HBM peak) + tokens/s at Qwen3-8B shape, batch 256",
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "global_batch": head["global_batch"],
                   "seq_len": head["seq_len"], "parallelism": "none (1 GPU)",
                   "block_size": head["block_size"], "pool_replicas": head["pool_replicas"],
                   "step_mode": head["step_mode"]},
    }
    for k in ("hbm_peak_frac", "tokens_per_s", "ms_per_call", "algorithmic_bytes", "roofline"):
        rec[k] = head[k]
    extra = {}
    if not args.only:
        for config in EXTRA_DECODE:
            if config == args.config:
                continue
            progress("%s decode" % config)
            extra[config] = run_decode(args, torch, B, W, dev, config,
                                       warmup=max(args.warmup, EXTRA_WARMUP),
                                       warm_s=EXTRA_WARMUP_S)
            torch.cuda.empty_cache()
        progress("prefill")
        extra["prefill"] = run_prefill(args, torch, B, W, dev,
                                       warmup=max(args.warmup, EXTRA_WARMUP),
                                       warm_s=EXTRA_WARMUP_S)
        torch.cuda.empty_cache()
        progress("36-layer step")
        rec["model_36_layers"] = run_model(args, torch, B, W, dev)
        torch.cuda.empty_cache()
    if args.mixed:
        progress("mixed")
        rec["mixed"] = run_mixed(args, torch, B, W, dev)
    if args.cpu_budget > 0:
        progress("CPU oracle baselines")
        rec["cpu_baseline"] = cpu_baseline(args, args.config)
        for config, obj in extra.items():
            obj["cpu_baseline"] = cpu_baseline(args, config)
    else:
        rec["cpu_baseline"] = None
    if extra:
        rec["configs"] = extra
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
