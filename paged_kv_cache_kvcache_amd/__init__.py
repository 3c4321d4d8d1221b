"""PagedAttention hot path for MI355X (gfx950): KV store, paged decode,
varlen prefill, behind the C-ABI library ``libpa.so``.

The binding functions load the library on first use and raise if it is
missing; nothing here falls back to a CPU implementation.
"""

from .binding import (  # noqa: F401
    LibraryNotBuilt,
    PAError,
    lib_path,
    load,
    pa_build_metadata,
    pa_decode,
    pa_decode_step,
    pa_decode_workspace_size,
    pa_mixed_varlen,
    pa_prefill_varlen,
    pa_store_kv,
)
