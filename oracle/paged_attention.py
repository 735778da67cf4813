"""The paged-attention reference: cache writes, block copies, decode and prefill chunks.

Everything is computed in float64 from the stored cache bits, by gathering
each token's K and V through the block table and running an explicit softmax.
"""

from __future__ import annotations

import numpy as np

from .layout import ELEM_BYTES, RAW_DTYPE, tile_positions
from .numerics import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode


# ----------------------------------------------------------------------------- sizes


def kv_bytes_per_token_page_formula(n_layers: int, n_heads: int, d_head: int, b_bytes: int) -> int:
    """KV-cache bytes per token as the equation on codebumble.net ("Technical Mechanics") prints
    it: 2 x 2 x n_layers x n_heads x d_head x b_bytes.  Kept verbatim, extra factor of 2 included;
    the physical size of a cache is kv_bytes_per_token_layer() x n_layers."""
    return 2 * 2 * n_layers * n_heads * d_head * b_bytes


def kv_bytes_per_token_per_layer_p3(head_size: int, num_heads: int, dtype_bytes: int) -> int:
    """Per-token, per-layer KV bytes as cyberpulstech.com's "Practical VRAM Math" settles on:
    (Head_Size x Num_Heads) x 2 (K and V) x Dtype_Bytes."""
    return head_size * num_heads * 2 * dtype_bytes


def kv_bytes_per_token_layer(Hkv: int, D: int, kv_dtype: str) -> int:
    """Bytes one token occupies in one layer's k_cache plus v_cache."""
    return 2 * Hkv * D * ELEM_BYTES[kv_dtype]


# ----------------------------------------------------------------------------- raw values


def new_cache(NB: int, Hkv: int, bs: int, D: int, kv_dtype: str) -> np.ndarray:
    """A zeroed raw cache [NB, Hkv, bs*D] (float32, bf16 bits as uint16, or fp8 codes)."""
    return np.zeros((NB, Hkv, bs * D), dtype=RAW_DTYPE[kv_dtype])


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "fp8":
        return e4m3fn_decode(raw)
    raise ValueError(dtype)


def encode_rows(x: np.ndarray, src_dtype: str, kv_dtype: str, scale: float) -> np.ndarray:
    """Source K or V rows -> the raw values the cache stores.

    f32 -> f32 and bf16 -> bf16 store the bits unchanged.  -> fp8 stores the
    e4m3fn code of the fp32 quotient x / scale (fp32 division, correctly rounded)."""
    if kv_dtype == src_dtype and kv_dtype in ("f32", "bf16"):
        return np.array(x, dtype=RAW_DTYPE[kv_dtype], copy=True)
    if kv_dtype == "fp8" and src_dtype in ("f32", "bf16"):
        x32 = to_f64(x, src_dtype).astype(np.float32)
        return e4m3fn_encode(x32 / np.float32(scale))
    raise ValueError(f"unsupported store {src_dtype} -> {kv_dtype}")


def slot_of(table_row: np.ndarray, positions, bs: int) -> np.ndarray:
    """Slot of token positions: logical block = position // bs and offset = position % bs
    (codebumble.net, "The Block Table Mapping Subsystem"), slot = frame * bs + offset."""
    positions = np.asarray(positions, dtype=np.int64)
    return np.asarray(table_row, dtype=np.int64)[positions // bs] * bs + positions % bs


# ----------------------------------------------------------------------------- cache writes


def reshape_and_cache(k_cache, v_cache, k, v, slot_mapping, *, bs: int, src_dtype: str,
                      kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                      batch: int = 2048) -> None:
    """Write token i's K and V rows ([Hkv, D] each) into slot slot_mapping[i] of the caches,
    in place: frame slot // bs, offset slot % bs.  Negative slots are skipped (padding).

    parity: bit-exact; pinned by tests against the diagram's block-table examples
    (logical blocks 0/1/2 at frames #14/#02/#89 and 41/08/93) and round trips."""
    T, Hkv, D = k.shape
    kpos = tile_positions("k", bs, D, kv_dtype)
    vpos = tile_positions("v", bs, D, kv_dtype)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    heads = np.arange(Hkv)[None, :, None]
    for s in range(0, T, batch):
        e = min(T, s + batch)
        sl = slots[s:e]
        ok = sl >= 0
        if not ok.any():
            continue
        f = (sl[ok] // bs)[:, None, None]
        o = sl[ok] % bs
        k_cache[f, heads, kpos[o][:, None, :]] = encode_rows(k[s:e][ok], src_dtype, kv_dtype, k_scale)
        v_cache[f, heads, vpos[o][:, None, :]] = encode_rows(v[s:e][ok], src_dtype, kv_dtype, v_scale)


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """Copy-on-write support (infoisland, section 2): frame dst := frame src for K and V, for
    every (src, dst) pair.  Destinations must be distinct and none may be a source, so the
    result does not depend on the order of the pairs.  parity: bit-exact."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if len(np.unique(dst)) != len(dst) or np.intersect1d(src, dst).size:
        raise ValueError("copy pairs need distinct destinations that are not sources")
    k_cache[dst] = k_cache[src]
    v_cache[dst] = v_cache[src]


# ----------------------------------------------------------------------------- attention


def gather_kv(cache, table_row, L: int, kind: str, *, bs: int, kv_dtype: str,
              scale: float = 1.0) -> np.ndarray:
    """[L, Hkv, D] float64 K (kind "k") or V of one sequence: token t is read from frame
    table_row[t // bs], slot t % bs, and dequantised (fp8 codes times the per-tensor scale)."""
    NB, Hkv, tile = cache.shape
    D = tile // bs
    pos = tile_positions(kind, bs, D, kv_dtype)
    t = np.arange(L)
    frame = np.asarray(table_row, dtype=np.int64)[t // bs]
    raw = cache[frame[:, None, None], np.arange(Hkv)[None, :, None], pos[t % bs][:, None, :]]
    vals = to_f64(raw, kv_dtype)
    if kv_dtype == "fp8":
        vals = vals * float(np.float32(scale))
    return vals


def _softmax_attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """qrows [R, D] against K, V [n, D]: softmax(scale * q.K^T) V with an explicit max shift."""
    s = scale * (K @ qrows.T)  # [n, R]
    s = s - s.max(axis=0, keepdims=True)
    p = np.exp(s)
    return (p.T @ V) / p.sum(axis=0)[:, None]


def decode(q, k_cache, v_cache, block_tables, context_lens, *, scale: float, bs: int,
           q_dtype: str, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
           seqs=None) -> np.ndarray:
    """Decode attention: for every sequence b and query head h (kv head g = h // G, G = Hq/Hkv),
    out[b, h] = sum_t softmax_t(scale * q[b, h] . K_b[t, g]) V_b[t, g] over t < context_lens[b],
    with K_b, V_b gathered through block_tables[b].  Returns float64 [len(seqs), Hq, D].

    parity: pinned (identity table = textbook attention via torch SDPA, frame-permutation
    invariance, one-token and identical-key closed forms, brute force on tiny inputs)."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    seqs = range(B) if seqs is None else seqs
    seqs = list(seqs)
    out = np.zeros((len(seqs), Hq, D))
    for n, b in enumerate(seqs):
        L = int(context_lens[b])
        K = gather_kv(k_cache, block_tables[b], L, "k", bs=bs, kv_dtype=kv_dtype, scale=k_scale)
        V = gather_kv(v_cache, block_tables[b], L, "v", bs=bs, kv_dtype=kv_dtype, scale=v_scale)
        qb = to_f64(q[b], q_dtype)
        for g in range(Hkv):
            out[n, g * G:(g + 1) * G] = _softmax_attend(qb[g * G:(g + 1) * G], K[:, g], V[:, g], scale)
    return out


def prefill_chunk(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, *,
                  scale: float, bs: int, q_dtype: str, kv_dtype: str, k_scale: float = 1.0,
                  v_scale: float = 1.0, rows=None) -> np.ndarray:
    """Causal attention of prefill chunks over their paged context.  Chunk c owns query rows
    r in [query_start_loc[c], query_start_loc[c+1]) (C rows); its sequence has L =
    context_lens[c] tokens including the chunk, so row i of the chunk sits at position
    L - C + i and attends keys 0 .. L - C + i inclusive.  Returns float64 [total_q, Hq, D];
    rows outside `rows` (if given) are left at zero.

    parity: pinned (one-row chunk = decode, chunk at position 0 with an identity table =
    causal SDPA, one chunk of 2n rows = two chunks of n)."""
    total_q, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    want = None if rows is None else set(int(r) for r in rows)
    out = np.zeros((total_q, Hq, D))
    for c in range(len(context_lens)):
        r0, r1 = int(qsl[c]), int(qsl[c + 1])
        C, L = r1 - r0, int(context_lens[c])
        mine = [r for r in range(r0, r1) if want is None or r in want]
        if not mine:
            continue
        K = gather_kv(k_cache, block_tables[c], L, "k", bs=bs, kv_dtype=kv_dtype, scale=k_scale)
        V = gather_kv(v_cache, block_tables[c], L, "v", bs=bs, kv_dtype=kv_dtype, scale=v_scale)
        for r in mine:
            pos = L - C + (r - r0)
            qr = to_f64(q[r], q_dtype)
            for g in range(Hkv):
                out[r, g * G:(g + 1) * G] = _softmax_attend(
                    qr[g * G:(g + 1) * G], K[:pos + 1, g], V[:pos + 1, g], scale)
    return out


def mixed_attention(q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                    num_decodes: int, *, scale: float, bs: int, q_dtype: str, kv_dtype: str,
                    k_scale: float = 1.0, v_scale: float = 1.0, rows=None) -> np.ndarray:
    """One step of a mixed batch: a prefill chunk and the ongoing decodes in the same iteration
    (bicarait.com, "Architectural Blueprint 3"; infoisland, section 5).  Sequences
    [0, num_decodes) are decodes, each with the single query row b (query_start_loc[b] = b); the
    others are chunks as in prefill_chunk.  A decode is its one query against its whole context,
    which is a chunk of one row at position L - 1, so the step is prefill_chunk over every
    sequence of the batch.  Returns float64 [total_q, Hq, D].

    parity: pinned (decode rows equal decode() on the decodes alone, chunk rows equal
    prefill_chunk() on the chunks alone)."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if num_decodes < 0 or np.any(qsl[:num_decodes + 1] != np.arange(num_decodes + 1)):
        raise ValueError("decode b must own query row b")
    return prefill_chunk(q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                         scale=scale, bs=bs, q_dtype=q_dtype, kv_dtype=kv_dtype, k_scale=k_scale,
                         v_scale=v_scale, rows=rows)
