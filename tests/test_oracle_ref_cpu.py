"""The whole-output oracle runner (tests/oracle_ref.py) assembles its pool
workers' pieces into exactly the oracle's single-process result."""

import os
import subprocess
import sys

import numpy as np

import oracle
import oracle_ref
from paged_kv_cache_kvcache_amd import workloads as W


def test_decode_pieces_equal_single_process():
    case = W.decode_case(8, 2, 64, [1, 0, 300, 17, 513, 256], seed=11)
    ref = oracle_ref.reference("decode", case)
    live = case.context_lens > 0
    slots = np.full(case.batch, -1, dtype=np.int32)
    slots[live] = oracle.build_metadata(case.block_tables[live], case.starts[live],
                                        case.context_lens[live], 256)[0]
    k, v = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    assert np.array_equal(ref, oracle.decode(case.q, k, v, case.block_tables, case.context_lens,
                                             case.scale))


def test_prefill_pieces_equal_single_process():
    case = W.prefill_case(8, 2, 64, 256, [1, 70, 130, 5], seed=12)
    ref = oracle_ref.reference("prefill", case)
    slots, cu_q, cu_k = oracle.build_metadata(case.block_tables, case.starts, case.ends, 256)
    k, v = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    assert np.array_equal(ref, oracle.prefill_varlen(case.q, k, v, cu_q, cu_k, case.block_tables,
                                                     case.scale))


def test_script_reports_errors_of_a_named_case(tmp_path):
    """The script end to end on the tiny workload: the oracle's own output
    rounded to bf16 is within half a bf16 ulp; an all-zero output is not."""
    case = W.make_case("tiny")
    ref = oracle_ref.reference("decode", case)
    good = W.round_to_bf16_bits(ref.astype(np.float32))
    for bits, ok in ((good, True), (np.zeros_like(good), False)):
        src, dst = tmp_path / "g.npy", tmp_path / "s.json"
        np.save(src, bits)
        subprocess.run([sys.executable, os.path.join(os.path.dirname(__file__), "oracle_ref.py"),
                        "decode", "tiny", str(src), str(dst)], check=True,
                       stdout=subprocess.DEVNULL)
        import json
        rec = json.loads(dst.read_text())
        assert rec["elements"] == ref.size
        if ok:
            assert rec["max_abs"] <= np.abs(ref).max() * 2.0 ** -8
        else:
            assert abs(rec["max_abs"] - np.abs(ref).max()) < 1e-12
