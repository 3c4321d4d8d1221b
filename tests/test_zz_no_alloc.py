"""GPU: pa_decode_noalloc (the decode entry point that allocates nothing; its
workspace is the library's per-GPU device array) through the C ABI, against
pa_decode on the same inputs, on two calls in a row, the second smaller,
and against the fp64 oracle (max-abs 1e-2, mean-abs 1e-3)."""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, dev_bf16, dev_i32, host_bits, host_f64
from paged_kv_cache_kvcache_amd import binding as B
from paged_kv_cache_kvcache_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _decode_both(case):
    """pa_decode (own workspace) and pa_decode_noalloc on the same inputs."""
    live = case.context_lens > 0
    slots = np.full(case.batch, -1, dtype=np.int32)  # padding rows store nothing
    slots[live] = B.pa_build_metadata(case.block_tables[live], case.starts[live],
                                      case.context_lens[live], case.block_size)[0]
    kc, vc = dev_bf16(case.k_cache), dev_bf16(case.v_cache)
    B.pa_store_kv(dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots))
    q = dev_bf16(case.q)
    bt, ctx = dev_i32(case.block_tables), dev_i32(case.context_lens)
    max_ctx = int(case.context_lens.max())
    out_ref = torch.empty_like(q)
    out_na = torch.full_like(q, float("nan"))
    B.pa_decode(q, kc, vc, bt, ctx, case.scale, out_ref, max_context_len=max_ctx)
    B.pa_decode_noalloc(q, kc, vc, bt, ctx, case.scale, out_na, max_context_len=max_ctx)
    torch.cuda.synchronize()
    kref, vref = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
    return host_bits(out_ref), host_bits(out_na), kref, vref


def test_noalloc_equals_decode_on_two_calls_second_smaller():
    # 1: 256 sequences (ordered grid, split-K partials in the scratch array);
    # 2: 40 shorter sequences right after, on the array the first call left
    for seed, lens in ((141, np.random.default_rng(140).integers(512, 8192 + 1, size=256)),
                       (143, np.random.default_rng(142).integers(1, 3000 + 1, size=40))):
        case = W.decode_case(32, 8, 128, lens, seed=seed)
        print("noalloc: %d seqs, max ctx %d, workspace %d bytes" % (
            case.batch, int(lens.max()),
            B.pa_decode_workspace_size(32, dev_bf16(case.k_cache[:1]), case.batch,
                                       int(lens.max()))), flush=True)
        ref_bits, na_bits, kref, vref = _decode_both(case)
        assert np.array_equal(na_bits, ref_bits), "pa_decode_noalloc differs from pa_decode"
        rows = sorted(set(range(0, case.batch, max(1, case.batch // 24))) | {case.batch - 1})
        ref = oracle.decode(case.q, kref, vref, case.block_tables, case.context_lens, case.scale,
                            rows=rows)
        got = oracle.bf16_bits_to_f64(na_bits)
        mx, mean = assert_close(got[rows], ref[rows], "noalloc %d seqs" % case.batch)
        print("  parity: max abs %.3g mean abs %.3g (rows %d)" % (mx, mean, len(rows)),
              flush=True)


def test_noalloc_matrix_core_path_and_padding_rows():
    lens = [0, 1, 300, 4097, 0, 2048]
    case = W.decode_case(64, 8, 128, lens, seed=144)
    ref_bits, na_bits, kref, vref = _decode_both(case)
    assert np.array_equal(na_bits, ref_bits)
    ref = oracle.decode(case.q, kref, vref, case.block_tables, case.context_lens, case.scale)
    assert_close(oracle.bf16_bits_to_f64(na_bits), ref, "noalloc mf")
    assert np.all(oracle.bf16_bits_to_f64(na_bits)[[0, 4]] == 0)
