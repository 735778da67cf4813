"""Plain CPU reference for paged attention (test infrastructure only).

This package is the oracle the GPU library is checked against.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
library and its Python binding never do.  It shares no code with the HIP path:
it decodes bf16 and fp8-e4m3fn bits itself, reads the cache tile layout from
its written definition, gathers K/V through the block table token by token and
runs an explicit fp64 softmax.

Sources (the pages this method is described on):
  * "Inside vLLM v0.7: How PagedAttention & Chunked Prefill Scaled 10x Token
    Serving" (bicarait.com), sections "Architectural Blueprint 2" (fixed-size
    blocks, block table, sharing) and "Architectural Blueprint 3" (chunked
    prefill).
  * "Inside vLLM Architecture: How PagedAttention and Continuous Batching
    Solved the KV Cache Crisis" (codebumble.net), sections "Technical
    Mechanics" (KV size per token), "Architectural Anatomy" (gather during
    QK^T), "The Block Table Mapping Subsystem" (slot = block, offset) and the
    FAQ answer that PagedAttention is exact.
  * cyberpulstech.com's "Practical VRAM Math" section (per-layer KV size).
  * "High-Throughput LLM Serving with vLLM & PagedAttention" (infoisland),
    sections 2 (copy-on-write), 4 (fp8 KV cache) and 5 (512-token chunks).

oracle.block_manager holds the reference model of the host block manager (free list,
on-demand allocation, fork, copy-on-write, release), pinned in tests/test_block_manager.py.

Parity status of each function is stated in its docstring; every function is
pinned by tests in tests/test_oracle.py against values the pages print,
closed forms, library routines on special cases or brute force.
"""

from .numerics import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3fn_table,
    e4m3fn_decode,
    e4m3fn_encode,
)
from .layout import ELEM_BYTES, tile_positions, pack_tiles, unpack_tiles  # noqa: F401
from .paged_attention import (  # noqa: F401
    kv_bytes_per_token_page_formula,
    kv_bytes_per_token_layer,
    kv_bytes_per_token_per_layer_p3,
    new_cache,
    encode_rows,
    reshape_and_cache,
    copy_blocks,
    gather_kv,
    decode,
    prefill_chunk,
    mixed_attention,
    slot_of,
)
from .block_manager import BlockManagerModel, OutOfBlocks  # noqa: F401
