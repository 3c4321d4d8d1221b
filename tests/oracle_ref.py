"""Whole-output oracle check of a named workload, in a process of its own.

The full-size workloads (256 x U[512, 8192] decode, 32 x 16,384 decode, the
18,342-query prefix-cached prefill, the mixed step) are checked on every
output row. The fp64 oracle needs tens of core-seconds for some of them, so
this script runs it in a fresh interpreter that never touches the GPU (the
test process has a GPU context and must not fork workers itself), in a pool
of forked worker processes, one per host core (at most 16):

    python tests/oracle_ref.py KIND CASE GPU_BITS OUT_JSON [--block-size B]

KIND is ``decode`` (store of each sequence's newest token, then decode) or
``prefill`` (store of the new tokens, then varlen prefill; the mixed step is
a prefill batch whose first rows have one query). The script redraws the
named CASE from its seed, derives the slots with the oracle's own metadata
builder, applies the oracle store, computes the oracle attention of every
row and compares it with the GPU output (bf16 bits in the .npy file
GPU_BITS). It writes the error statistics to OUT_JSON. Test
infrastructure only: it imports the oracle and the input generators.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from paged_kv_cache_kvcache_amd import workloads as W  # noqa: E402

_STATE = {}


def _decode_rows(rows):
    c, kref, vref = _STATE["case"], _STATE["k"], _STATE["v"]
    return rows, np.stack([oracle.decode_one(c.q[b], kref, vref, c.block_tables[b],
                                             int(c.context_lens[b]), c.scale) for b in rows])


def _prefill_piece(task):
    b, lo, hi = task
    c, kref, vref, cu_q = _STATE["case"], _STATE["k"], _STATE["v"], _STATE["cu_q"]
    q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
    r = oracle.prefill_one(c.q[q0:q1], kref, vref, c.block_tables[b], int(c.ends[b]), c.scale,
                           query_rows=range(lo, hi))
    return q0 + lo, r[lo:hi]


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def reference(kind: str, case) -> np.ndarray:
    """The oracle's output for every row of the case (float64), computed in
    a fork pool (the caller must be a process without a GPU context)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    if kind == "decode":
        ends = case.context_lens
        live = ends > 0
        slots = np.full(case.batch, -1, dtype=np.int32)
        slots[live] = oracle.build_metadata(case.block_tables[live], case.starts[live],
                                            ends[live], case.block_size)[0]
        cu_q = None
    else:
        slots, cu_q, _ = oracle.build_metadata(case.block_tables, case.starts, case.ends,
                                               case.block_size)
    kref, vref = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    _STATE.update(case=case, k=kref, v=vref, cu_q=cu_q)
    out = np.zeros(case.q.shape, dtype=np.float64)
    if kind == "decode":
        # longest sequences first, a few per task
        order = np.argsort(-case.context_lens, kind="stable").tolist()
        tasks = [order[i:i + 2] for i in range(0, len(order), 2)]
        fn = _decode_rows
    else:
        tasks = []
        for b in range(case.batch):
            n = int(cu_q[b + 1] - cu_q[b])
            step = 64
            tasks += [(b, lo, min(n, lo + step)) for lo in range(0, n, step)]
        # the pieces with the most visible keys first
        tasks.sort(key=lambda t: -(int(case.ends[t[0]]) - int(cu_q[t[0] + 1] - cu_q[t[0]]) + t[2]))
        fn = _prefill_piece
    with threadpool_limits(1):
        with mp.get_context("fork").Pool(workers()) as pool:
            for key, val in pool.imap_unordered(fn, tasks):
                if kind == "decode":
                    out[key] = val
                else:
                    out[key:key + len(val)] = val
    return out


def compare(got_bits: np.ndarray, ref: np.ndarray) -> dict:
    got = oracle.bf16_bits_to_f64(got_bits)
    finite = bool(np.all(np.isfinite(got)))
    err = np.abs(got - ref)
    i = int(np.nanargmax(err)) if finite else int(np.argmax(~np.isfinite(got).reshape(-1)))
    idx = np.unravel_index(i, ref.shape)
    return {"finite": finite, "max_abs": float(np.nanmax(err)), "mean_abs": float(np.nanmean(err)),
            "argmax": [int(x) for x in idx], "got_at_max": float(got[idx]),
            "ref_at_max": float(ref[idx]), "max_abs_ref": float(np.abs(ref).max()),
            "elements": int(ref.size)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["decode", "prefill"])
    ap.add_argument("case")
    ap.add_argument("gpu_bits")
    ap.add_argument("out_json")
    ap.add_argument("--block-size", type=int, default=W.BLOCK_SIZE)
    args = ap.parse_args()
    t0 = time.perf_counter()
    case = W.make_case(args.case, block_size=args.block_size)
    print("oracle_ref: %s %s drawn in %.1f s" % (args.kind, args.case, time.perf_counter() - t0),
          flush=True)
    ref = reference(args.kind, case)
    got = np.load(args.gpu_bits, allow_pickle=False)
    if got.shape != ref.shape:
        raise SystemExit("shape %s != %s" % (got.shape, ref.shape))
    rec = compare(got, ref)
    rec.update(kind=args.kind, case=args.case, block_size=args.block_size,
               workers=workers(), seconds=round(time.perf_counter() - t0, 2))
    with open(args.out_json, "w") as f:
        json.dump(rec, f)
    print("oracle_ref: %s" % json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
