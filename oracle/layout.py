"""The cache tile layout, read from its written definition.

k_cache and v_cache each hold NB frames of Hkv tiles; tile (f, g) holds the bs
tokens of frame f for kv head g.  The pages fix only that a frame holds a
fixed number of tokens (16 or 32) whose keys and values a kernel fetches
together (codebumble.net, "CUDA Shared Memory Optimization": a 16-token block
in an aligned structure, fetched with coalesced transactions); the order of
the bs x D values inside a tile is this library's choice and is defined in
include/pa.h.  With b bytes per element, token slot o and head-dim index d:

  K:  h = o // 16, kl = o % 16, j = d // (D/4), t = d % (D/4)
      byte = 1024 * (h * (D*b/64) + (t*b) // 16) + 16 * (16*j + kl) + (t*b) % 16
  V:  h = o // 16, j = (o % 16) // 4, i = o % 4, c = d // 16, dl = d % 16,
      u = h * (D/16) + c, Q = 4 / b
      byte = 1024 * (u // Q) + 16 * (16*j + dl) + (4 * (u % Q) + i) * b

The functions below evaluate these formulas one (o, d) pair at a time.
"""

from __future__ import annotations

from functools import lru_cache

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
RAW_DTYPE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def _k_byte(o: int, d: int, bs: int, D: int, b: int) -> int:
    h, kl = o // 16, o % 16
    j, t = d // (D // 4), d % (D // 4)
    loads_per_group = D * b // 64
    return 1024 * (h * loads_per_group + (t * b) // 16) + 16 * (16 * j + kl) + (t * b) % 16


def _v_byte(o: int, d: int, bs: int, D: int, b: int) -> int:
    h, j, i = o // 16, (o % 16) // 4, o % 4
    c, dl = d // 16, d % 16
    u = h * (D // 16) + c
    Q = 4 // b
    return 1024 * (u // Q) + 16 * (16 * j + dl) + (4 * (u % Q) + i) * b


@lru_cache(maxsize=None)
def tile_positions(kind: str, bs: int, D: int, dtype: str) -> np.ndarray:
    """[bs, D] array: element index inside a tile of the value for (slot o, dim d)."""
    b = ELEM_BYTES[dtype]
    fn = _k_byte if kind == "k" else _v_byte
    pos = np.empty((bs, D), dtype=np.int64)
    for o in range(bs):
        for d in range(D):
            byte = fn(o, d, bs, D, b)
            assert byte % b == 0
            pos[o, d] = byte // b
    assert np.array_equal(np.sort(pos.ravel()), np.arange(bs * D)), "layout is not a bijection"
    pos.setflags(write=False)
    return pos


def pack_tiles(values: np.ndarray, kind: str, dtype: str) -> np.ndarray:
    """values [..., bs, D] (raw element arrays) -> tiles [..., bs*D] in the cache layout."""
    bs, D = values.shape[-2:]
    pos = tile_positions(kind, bs, D, dtype)
    out = np.empty(values.shape[:-2] + (bs * D,), dtype=values.dtype)
    out[..., pos.ravel()] = values.reshape(values.shape[:-2] + (bs * D,))
    return out


def unpack_tiles(tiles: np.ndarray, kind: str, dtype: str, bs: int, D: int) -> np.ndarray:
    """tiles [..., bs*D] in the cache layout -> values [..., bs, D]."""
    pos = tile_positions(kind, bs, D, dtype)
    return tiles[..., pos.ravel()].reshape(tiles.shape[:-1] + (bs, D))
