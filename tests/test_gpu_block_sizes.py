"""GPU parity at block sizes other than 256 (powers of two 16..1024): the
same two-step slot map and the same attention, so store, decode, the fused
step and prefill must match the fp64 oracle at every block size (store
bit-exact; attention max-abs 1e-2 / mean-abs 1e-3). Small blocks are the
case where one load group or one 64-key stage spans several blocks."""

import numpy as np
import pytest

import oracle
from gpu_helpers import (assert_close, check_whole_output, dev_bf16, dev_i32, host_bits, host_f64,
                         poison_unused)
from paged_kv_cache_kvcache_amd import binding as B
from paged_kv_cache_kvcache_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BLOCK_SIZES = [16, 32, 64, 128, 512, 1024]
# lengths around multiples of every block size and of the 32/64-token chunks
LENS = [1, 15, 16, 17, 33, 63, 64, 65, 255, 257, 511, 513, 1023, 1025, 2049, 3000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _slots(case, ends):
    slots, _, _ = B.pa_build_metadata(case.block_tables, case.starts, ends, case.block_size)
    full = np.full(case.batch, -1, dtype=np.int32)
    full[ends > 0] = slots
    return full


@pytest.mark.parametrize("bsz", BLOCK_SIZES)
@pytest.mark.parametrize("h_q,h_kv,d", [(32, 8, 128), (8, 1, 64), (64, 8, 128), (32, 8, 64)])
def test_store_and_decode(bsz, h_q, h_kv, d):
    case = W.decode_case(h_q, h_kv, d, LENS, seed=90 + bsz + d, block_size=bsz)
    print("block size %d decode H=%d/%d d=%d pool=%d blocks" % (bsz, h_q, h_kv, d,
                                                               case.num_blocks), flush=True)
    slots = _slots(case, case.context_lens)
    kc0, vc0 = poison_unused(case.k_cache, case.v_cache, case.block_tables, case.starts, bsz)
    kc, vc = dev_bf16(kc0), dev_bf16(vc0)
    B.pa_store_kv(dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots))
    q = dev_bf16(case.q)
    out = torch.empty_like(q)
    B.pa_decode(q, kc, vc, dev_i32(case.block_tables), dev_i32(case.context_lens), case.scale,
                out, max_context_len=int(case.context_lens.max()))
    torch.cuda.synchronize()
    kref, vref = oracle.store_kv(kc0, vc0, case.k_new, case.v_new, slots)
    assert np.array_equal(host_bits(kc), kref) and np.array_equal(host_bits(vc), vref)
    ref = oracle.decode(case.q, kref, vref, case.block_tables, case.context_lens, case.scale)
    mx, mean = assert_close(host_f64(out), ref, "decode B=%d" % bsz)
    print("  parity: max abs %.3g mean abs %.3g" % (mx, mean), flush=True)


@pytest.mark.parametrize("bsz", [16, 64, 1024])
@pytest.mark.parametrize("h_q,h_kv,d", [(32, 8, 128), (16, 4, 64), (64, 4, 128), (40, 8, 128),
                                         (32, 4, 64)])
def test_fused_step(bsz, h_q, h_kv, d):
    case = W.decode_case(h_q, h_kv, d, LENS, seed=95 + bsz, block_size=bsz)
    print("block size %d fused step" % bsz, flush=True)
    slots = _slots(case, case.context_lens)
    kc0, vc0 = poison_unused(case.k_cache, case.v_cache, case.block_tables, case.starts, bsz)
    kc, vc = dev_bf16(kc0), dev_bf16(vc0)
    q = dev_bf16(case.q)
    out = torch.empty_like(q)
    B.pa_decode_step(q, dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots),
                     dev_i32(case.block_tables), dev_i32(case.context_lens), case.scale, out,
                     max_context_len=int(case.context_lens.max()))
    torch.cuda.synchronize()
    kref, vref = oracle.store_kv(kc0, vc0, case.k_new, case.v_new, slots)
    assert np.array_equal(host_bits(kc), kref) and np.array_equal(host_bits(vc), vref)
    ref = oracle.decode(case.q, kref, vref, case.block_tables, case.context_lens, case.scale)
    assert_close(host_f64(out), ref, "fused step B=%d" % bsz)


def _prefill_case(h_q, h_kv, d, bsz, seed):
    """Cached prefixes that end anywhere in a block, ragged suffixes."""
    rng = np.random.default_rng(seed)
    starts = np.array([0, 3, 16, 40, 300, 511, 700, 64], dtype=np.int32)
    suffix = np.array([70, 1, 15, 129, 2, 300, 33, 64], dtype=np.int32)
    ends = starts + suffix
    need = [W.blocks_needed(int(e), bsz) for e in ends]
    nb = int(np.ceil(1.1 * sum(need)))
    perm = rng.permutation(nb)
    tables, pos = [], 0
    for n in need:
        tables.append(perm[pos:pos + n].tolist())
        pos += n
    total = int(suffix.sum())
    return W.PrefillCase("ragged B=%d" % bsz, h_q, h_kv, d, bsz, nb,
                         W.normal_bf16(rng, (total, h_q, d)),
                         W.normal_bf16(rng, (total, h_kv, d)),
                         W.normal_bf16(rng, (total, h_kv, d)),
                         W.normal_bf16(rng, (nb, bsz, h_kv, d)),
                         W.normal_bf16(rng, (nb, bsz, h_kv, d)),
                         W.pad_tables(tables), starts, ends, 1.0 / np.sqrt(d), seed)


@pytest.mark.parametrize("bsz", BLOCK_SIZES)
@pytest.mark.parametrize("h_q,h_kv,d", [(32, 8, 128), (16, 2, 64)])
def test_prefill(bsz, h_q, h_kv, d):
    case = _prefill_case(h_q, h_kv, d, bsz, seed=97 + bsz + d)
    print("block size %d prefill H=%d/%d d=%d" % (bsz, h_q, h_kv, d), flush=True)
    slots, cu_q, cu_k = B.pa_build_metadata(case.block_tables, case.starts, case.ends, bsz)
    kc0, vc0 = poison_unused(case.k_cache, case.v_cache, case.block_tables, case.starts, bsz)
    kc, vc = dev_bf16(kc0), dev_bf16(vc0)
    B.pa_store_kv(dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots))
    q = dev_bf16(case.q)
    out = torch.empty_like(q)
    qlens = case.ends - case.starts
    B.pa_prefill_varlen(q, kc, vc, dev_i32(cu_q), dev_i32(cu_k), int(qlens.max()),
                        int(case.ends.max()), dev_i32(case.block_tables), case.scale, out)
    torch.cuda.synchronize()
    kref, vref = oracle.store_kv(kc0, vc0, case.k_new, case.v_new, slots)
    assert np.array_equal(host_bits(kc), kref) and np.array_equal(host_bits(vc), vref)
    ref = oracle.prefill_varlen(case.q, kref, vref, cu_q, cu_k, case.block_tables, case.scale)
    mx, mean = assert_close(host_f64(out), ref, "prefill B=%d" % bsz)
    print("  parity: max abs %.3g mean abs %.3g" % (mx, mean), flush=True)


def test_qwen3_8b_shape_at_block_16():
    """The 256-sequence Qwen3-8B decode batch with 16-token blocks (16x the
    table entries); every row vs the oracle (computed in a separate
    process)."""
    case = W.make_case("qwen3-8b", block_size=16)
    print("block size 16 qwen3-8b shape: %d blocks" % case.num_blocks, flush=True)
    slots, _, _ = B.pa_build_metadata(case.block_tables, case.starts, case.context_lens, 16)
    kc, vc = dev_bf16(case.k_cache), dev_bf16(case.v_cache)
    B.pa_store_kv(dev_bf16(case.k_new), dev_bf16(case.v_new), kc, vc, dev_i32(slots))
    q = dev_bf16(case.q)
    out = torch.empty_like(q)
    B.pa_decode(q, kc, vc, dev_i32(case.block_tables), dev_i32(case.context_lens), case.scale,
                out, max_context_len=int(case.context_lens.max()))
    torch.cuda.synchronize()
    del kc, vc
    check_whole_output("decode", "qwen3-8b", out, block_size=16)
