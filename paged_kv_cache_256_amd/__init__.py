"""MI355X-native paged attention: hand-written gfx950 HIP kernels behind a C ABI (libpa.so).

The Python layer only marshals torch tensors (device memory, streams) into the C entry points
declared in include/pa.h:

    reshape_and_cache  write this step's K/V rows into their cache slots
    copy_blocks        duplicate frames for copy-on-write
    decode             paged GQA decode attention (split over the context + reduce)
    decode_noalloc     the same decode on the library's own device scratch (allocates nothing)
    decode_shared      decode reading a run's shared prompt frames once for all its members
    prefill_chunk      causal attention of prefill chunks over their paged context
    mixed_attention    decodes and prefill chunks of one step in one persistent kernel
    BlockManager       host-side frames, block tables, slots and copy-on-write pairs
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    BlockManager,
    LIB_PATH,
    PAError,
    PreparedCall,
    build_info,
    copy_blocks,
    decode,
    decode_noalloc,
    decode_shared,
    decode_shared_workspace_bytes,
    decode_workspace_bytes,
    find_shared_prefixes,
    SharedRuns,
    SHARED_RUN_COLUMNS,
    last_error,
    lib,
    mixed_attention,
    mixed_prefill_units,
    mixed_workspace_bytes,
    new_kv_cache,
    prefill_chunk,
    prefill_chunk_workspace_bytes,
    q_dtype_for,
    reshape_and_cache,
    validate_chunk_indices,
    validate_copy_pairs,
    validate_decode_indices,
    validate_mixed_indices,
    validate_shared_prefixes,
    validate_slots,
)
