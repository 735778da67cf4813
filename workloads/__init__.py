"""Seeded synthetic inputs for the paged-attention workloads.

This package is shared by the tests, the benchmark and the checks of the CPU
reference.  It holds random draws and bookkeeping only: sequence lengths, the
assignment of logical blocks to physical frames, slot lists, fork/copy-on-write
bookkeeping and poison values.  It holds no attention arithmetic, no cache
layout and no quantisation; those live on each side of the comparison
separately.
"""

from .cases import (  # noqa: F401
    DecodeCase,
    ChunkPart,
    make,
    decode_case,
    chunk_case,
    config5_variant,
    long_context,
    fork_case,
    mixed_batch,
    MixedBatch,
    CONFIG_NAMES,
    POISON_K,
    POISON_V,
    SCORE_PROFILES,
    steer_scores,
)
