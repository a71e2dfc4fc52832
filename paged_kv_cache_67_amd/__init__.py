"""paged_kv_cache_67_amd -- paged attention over a block-managed KV cache on MI355X.

The compute path is ``libpa.so`` (hand-written HIP for gfx950, C ABI in
``include/pa.h``); this package is its thin Python binding plus a host-side
harness that lays a synthetic workload out in device memory and enqueues one
step of the path.  Importing the package does not load the library; the first
call does, and fails loudly if it has not been built.
"""

from ._binding import (  # noqa: F401
    PA_BF16,
    PA_F16,
    PA_F32,
    BlockManager,
    PAError,
    lib,
    lib_path,
    pa_attention_mixed,
    pa_chain_hash,
    pa_check_decode_inputs,
    pa_check_prefill_inputs,
    pa_check_store_inputs,
    pa_check_store_paged_inputs,
    pa_copy_blocks,
    pa_copy_many,
    pa_read_ceiling,
    pa_decode,
    pa_decode_append,
    pa_decode_append_partitions,
    pa_decode_merge,
    pa_decode_noalloc,
    pa_decode_partitions,
    pa_decode_workspace_size,
    pa_last_error,
    pa_mixed_workspace_size,
    pa_prefill_paged,
    pa_set_debug_checks,
    pa_slot_mapping,
    pa_status_string,
    pa_store_kv,
    pa_store_kv_paged,
    pa_version,
)
