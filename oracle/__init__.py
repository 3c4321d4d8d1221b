"""Plain, slow CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY. This package is imported by the test suite, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
nothing in the product package (``paged_kv_cache_kvcache_amd``) may import or
call it. It shares no code with the HIP path: it imports numpy and nothing
else, and receives the same seeded input arrays (bf16 bit patterns as uint16,
int32 metadata) that the GPU path receives.

All floating point is IEEE float64. bf16 inputs are widened exactly.

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself: the worked examples printed on the pages, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64) on the
special case of an identity block table, closed forms and invariants.
"""

from .paged_attention import (  # noqa: F401
    bf16_bits_to_f64,
    slot_of,
    slots_for_range,
    decode_slot,
    cu_seqlens,
    build_metadata,
    store_kv,
    gather_rows,
    used_rows,
    decode,
    decode_one,
    prefill_varlen,
    prefill_one,
)
