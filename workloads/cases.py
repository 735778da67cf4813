"""Seeded synthetic paged-attention inputs.

Every case is built from one numpy PCG64 generator in a fixed draw order:
context lengths, then the frame permutation, then q, the K pool, the V pool,
the new K rows and the new V rows.  Values are drawn in fp32 and, for bf16
inputs, rounded to bf16 (round to nearest even) by torch's cast.

Bookkeeping conventions (the ABI's encoding of its index inputs):
  * a sequence of context length L occupies logical blocks 0..ceil(L/bs)-1;
  * logical block i of sequence b lives in physical frame block_tables[b, i];
    unused table entries are -1;
  * the slot of token position t is frame * bs + t % bs with
    frame = block_tables[b, t // bs];
  * context_lens count the tokens written in this step (a decode step writes
    position L-1 before attending; a prefill chunk of C tokens writes
    positions L-C .. L-1).

Slots that hold no live token before the step (unused frames, the tail of a
sequence's last frame, the slots this step writes, copy-on-write targets) are
filled with poison values so that a kernel that reads them where it must not,
or skips a write it must make, produces a visibly wrong result.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

POISON_K = 30.0
POISON_V = 1000.0

CONFIG_NAMES = {
    1: "tiny-f32-decode B4 Hq4 Hkv2 D64 bs16",
    2: "llama3-8b-decode bf16 B64 Hq32 Hkv8 D128 bs16",
    3: "llama3-70b-decode bf16 B256 Hq64 Hkv8 D128 bs16",
    4: "llama3-70b-decode fp8-kv bs32 32 prompts x 8 branches (cow)",
    5: "llama3-8b-mixed chunk512@16384 + 128 decodes bf16 bs16",
}

_CHUNK_ROWS = 1 << 22  # values drawn per numpy call (bounds host memory)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) values of `shape`, as float32 or bf16 bit patterns (uint16)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    std32 = np.float32(std)
    for s in range(0, n, _CHUNK_ROWS):
        e = min(n, s + _CHUNK_ROWS)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= std32
        out[s:e] = x if dtype == "f32" else _bf16_bits(x)
    return out.reshape(shape)


def _const(value: float, dtype: str):
    if dtype == "f32":
        return np.float32(value)
    return _bf16_bits(np.array([value], dtype=np.float32))[0]


def _as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclass
class ChunkPart:
    """Prefill chunks of a mixed step: query rows [query_start_loc[c], query_start_loc[c+1])
    of `q` belong to chunk c, whose sequence has context_lens[c] tokens including the chunk."""

    q: np.ndarray  # [total_q, Hq, D]
    query_start_loc: np.ndarray  # int32 [num_chunks + 1]
    context_lens: np.ndarray  # int32 [num_chunks]
    block_tables: np.ndarray  # int32 [num_chunks, max_blocks]
    new_rows: slice  # rows of the case's new_k/new_v/new_slots that are the chunks' tokens

    @property
    def num_chunks(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_chunk_len(self) -> int:
        return int(np.max(np.diff(self.query_start_loc))) if self.num_chunks else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_chunks else 0


@dataclass
class DecodeCase:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    q_dtype: str  # "f32" | "bf16"
    kv_dtype: str  # "f32" | "bf16" | "fp8"
    src_dtype: str  # dtype of pool / new K,V rows: "f32" | "bf16"
    scale: float
    k_scale: float
    v_scale: float
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    q: np.ndarray  # [B, Hq, D]
    pool_k: np.ndarray  # [NB*bs, Hkv, D] value held at every slot before the step
    pool_v: np.ndarray
    new_k: np.ndarray  # [T, Hkv, D]
    new_v: np.ndarray
    new_slots: np.ndarray  # int64 [T]
    copy_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int64))
    chunk: ChunkPart | None = None
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def pool_slots(self) -> np.ndarray:
        return np.arange(self.NB * self.bs, dtype=np.int64)

    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    @property
    def shares_frames(self) -> bool:
        """True if some frame appears in the used block-table entries of two decode sequences
        (the caller's hint that frames are shared within the batch)."""
        if not self.B:
            return False
        nblk = (self.context_lens.astype(np.int64) + self.bs - 1) // self.bs
        used = np.concatenate([self.block_tables[b, :n] for b, n in enumerate(nblk)])
        return bool(np.unique(used).size < used.size)

    def decode_kv_bytes(self, seqs=None) -> int:
        """Algorithmic KV bytes a decode step must read: L * 2 * Hkv * D * b per sequence."""
        lens = self.context_lens if seqs is None else self.context_lens[seqs]
        return int(np.sum(lens.astype(np.int64))) * 2 * self.Hkv * self.D * self.kv_elem_bytes()


# ----------------------------------------------------------------------------- helpers


def _assign_tables(perm: np.ndarray, nblk: np.ndarray, start: int = 0, width: int | None = None):
    """Consecutive entries of `perm` (from `start`) go to sequence 0's blocks, then 1's, ..."""
    width = int(nblk.max()) if width is None else width
    tables = np.full((len(nblk), max(width, 1)), -1, dtype=np.int32)
    off = start
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[off : off + n]
        off += n
    return tables, off


def _slots(table_row: np.ndarray, positions: np.ndarray, bs: int) -> np.ndarray:
    return table_row[positions // bs].astype(np.int64) * bs + positions % bs


def _poison(pool_k, pool_v, live: np.ndarray, src_dtype: str):
    pool_k[~live] = _const(POISON_K, src_dtype)
    pool_v[~live] = _const(POISON_V, src_dtype)


def _fp8_scales(pool_k, pool_v, live, new_k, new_v, src_dtype):
    """Per-tensor scales: amax over every real (non-poison) K (V) value, divided by 448, in fp32."""
    ak = max(float(np.abs(_as_f32(pool_k[live], src_dtype)).max(initial=0.0)),
             float(np.abs(_as_f32(new_k, src_dtype)).max(initial=0.0)))
    av = max(float(np.abs(_as_f32(pool_v[live], src_dtype)).max(initial=0.0)),
             float(np.abs(_as_f32(new_v, src_dtype)).max(initial=0.0)))
    ks = np.float32(ak) / np.float32(448.0)
    vs = np.float32(av) / np.float32(448.0)
    return float(ks if ks > 0 else np.float32(1.0)), float(vs if vs > 0 else np.float32(1.0))


# ----------------------------------------------------------------------------- builders


def decode_case(name: str, seed: int, *, Hq: int, Hkv: int, D: int, bs: int, lens,
                kv_dtype: str = "bf16", q_dtype: str | None = None, std: float = 1.0,
                pool: str | int = "exact", lens_rng=None) -> DecodeCase:
    """A decode step over B sequences: each writes its token at position L-1, then attends.

    lens: array of context lengths, or a callable rng -> lengths (drawn first).
    pool: "exact" (NB = total blocks), "scattered" (NB = ceil(1.25 * total)), or an int NB.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng) if callable(lens) else lens, dtype=np.int64)
    B = len(lens)
    src = "f32" if kv_dtype == "f32" else "bf16"
    q_dtype = q_dtype or src
    nblk = -(-lens // bs)
    total = int(nblk.sum())
    if pool == "exact":
        NB = total
    elif pool == "scattered":
        NB = int(math.ceil(1.25 * total))
    else:
        NB = int(pool)
    assert NB >= total
    perm = rng.permutation(NB)
    tables, _ = _assign_tables(perm, nblk)
    q = _draw(rng, (B, Hq, D), std, q_dtype)
    pool_k = _draw(rng, (NB * bs, Hkv, D), std, src)
    pool_v = _draw(rng, (NB * bs, Hkv, D), std, src)
    new_k = _draw(rng, (B, Hkv, D), std, src)
    new_v = _draw(rng, (B, Hkv, D), std, src)
    live = np.zeros(NB * bs, dtype=bool)
    new_slots = np.empty(B, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        live[_slots(tables[b], np.arange(L - 1), bs)] = True
        new_slots[b] = _slots(tables[b], np.array([L - 1]), bs)[0]
    _poison(pool_k, pool_v, live, src)
    ks, vs = (1.0, 1.0)
    if kv_dtype == "fp8":
        ks, vs = _fp8_scales(pool_k, pool_v, live, new_k, new_v, src)
    return DecodeCase(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
                      q_dtype=q_dtype, kv_dtype=kv_dtype, src_dtype=src,
                      scale=1.0 / math.sqrt(D), k_scale=ks, v_scale=vs,
                      context_lens=lens.astype(np.int32), block_tables=tables, q=q,
                      pool_k=pool_k, pool_v=pool_v, new_k=new_k, new_v=new_v,
                      new_slots=new_slots, meta={"live_slots": int(live.sum())})


def chunk_case(name: str, seed: int, *, Hq: int, Hkv: int, D: int, bs: int, chunks,
               decode_lens=(), kv_dtype: str = "bf16", std: float = 1.0) -> DecodeCase:
    """A mixed step: prefill chunks (each a (chunk_len C, context_len L) pair; the chunk holds
    positions L-C..L-1 and writes them this step) plus decode sequences (context lengths, or a
    callable rng -> lengths drawn first).  One shuffled pool holds every sequence, chunk
    sequences first."""
    rng = np.random.default_rng(seed)
    dl = np.asarray(decode_lens(rng) if callable(decode_lens) else decode_lens, dtype=np.int64)
    chunks = [(int(c), int(L)) for c, L in chunks]
    src = "f32" if kv_dtype == "f32" else "bf16"
    clen = np.array([L for _, L in chunks], dtype=np.int64)
    cnew = np.array([c for c, _ in chunks], dtype=np.int64)
    all_lens = np.concatenate([clen, dl])
    nblk = -(-all_lens // bs)
    NB = int(nblk.sum())
    perm = rng.permutation(NB)
    width = int(nblk.max()) if len(nblk) else 1
    tables_all, _ = _assign_tables(perm, nblk, width=width)
    nc = len(chunks)
    q_dec = _draw(rng, (len(dl), Hq, D), std, src)
    q_chunk = _draw(rng, (int(cnew.sum()), Hq, D), std, src)
    pool_k = _draw(rng, (NB * bs, Hkv, D), std, src)
    pool_v = _draw(rng, (NB * bs, Hkv, D), std, src)
    T = int(cnew.sum()) + len(dl)
    new_k = _draw(rng, (T, Hkv, D), std, src)
    new_v = _draw(rng, (T, Hkv, D), std, src)
    live = np.zeros(NB * bs, dtype=bool)
    new_slots = []
    n_new = np.concatenate([cnew, np.ones(len(dl), dtype=np.int64)])
    for s in range(len(all_lens)):
        L, n = int(all_lens[s]), int(n_new[s])
        live[_slots(tables_all[s], np.arange(L - n), bs)] = True
        new_slots.append(_slots(tables_all[s], np.arange(L - n, L), bs))
    _poison(pool_k, pool_v, live, src)
    qsl = np.zeros(nc + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(cnew)
    chunk = ChunkPart(q=q_chunk, query_start_loc=qsl, context_lens=clen.astype(np.int32),
                      block_tables=tables_all[:nc].copy(), new_rows=slice(0, int(cnew.sum())))
    ks, vs = (1.0, 1.0)
    if kv_dtype == "fp8":
        ks, vs = _fp8_scales(pool_k, pool_v, live, new_k, new_v, src)
    return DecodeCase(name=name, seed=seed, B=len(dl), Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
                      q_dtype=src, kv_dtype=kv_dtype, src_dtype=src, scale=1.0 / math.sqrt(D),
                      k_scale=ks, v_scale=vs, context_lens=dl.astype(np.int32),
                      block_tables=tables_all[nc:].copy(), q=q_dec, pool_k=pool_k,
                      pool_v=pool_v, new_k=new_k, new_v=new_v,
                      new_slots=np.concatenate(new_slots) if new_slots else np.zeros(0, np.int64),
                      chunk=chunk, meta={"live_slots": int(live.sum())})


@dataclass
class MixedBatch:
    """A case's decodes and prefill chunks as one batch, decodes first: query row b is decode b,
    the chunks' rows follow; query_start_loc, context_lens and block_tables cover every
    sequence of the batch."""

    q: np.ndarray  # [B + chunk rows, Hq, D]
    query_start_loc: np.ndarray  # int32 [B + num_chunks + 1]
    context_lens: np.ndarray  # int32 [B + num_chunks]
    block_tables: np.ndarray  # int32 [B + num_chunks, width]
    num_decodes: int
    decode_tokens: int  # sum of the decodes' context lengths
    max_chunk_len: int
    max_context_len: int


def mixed_batch(case: DecodeCase) -> MixedBatch:
    """Concatenate the decodes and the chunks of `case` (bookkeeping only)."""
    B, ch = case.B, case.chunk
    nc = ch.num_chunks if ch is not None else 0
    parts = [case.block_tables[:B]] + ([ch.block_tables] if nc else [])
    width = max(max(p.shape[1] for p in parts), 1)
    tables = np.full((B + nc, width), -1, dtype=np.int32)
    tables[:B, :case.block_tables.shape[1]] = case.block_tables[:B]
    if nc:
        tables[B:, :ch.block_tables.shape[1]] = ch.block_tables
    q = np.concatenate([case.q[:B]] + ([ch.q] if nc else []), axis=0)
    qsl = np.arange(B + 1, dtype=np.int32)
    if nc:
        qsl = np.concatenate([qsl[:B], B + ch.query_start_loc.astype(np.int32)])
    lens = np.concatenate([case.context_lens[:B]] + ([ch.context_lens] if nc else [])).astype(np.int32)
    return MixedBatch(q=q, query_start_loc=qsl.astype(np.int32), context_lens=lens,
                      block_tables=tables, num_decodes=B,
                      decode_tokens=int(case.context_lens[:B].astype(np.int64).sum()),
                      max_chunk_len=ch.max_chunk_len if nc else 0,
                      max_context_len=int(lens.max()) if len(lens) else 1)


def fork_case(name: str, seed: int, *, prompts: int = 32, branches: int = 8,
              prompt_len: int = 1024, tail_lo: int = 64, tail_hi: int = 512, Hq: int = 64,
              Hkv: int = 8, D: int = 128, bs: int = 32, kv_dtype: str = "fp8",
              std: float = 1.0 / math.sqrt(2.0), spare: int = 64) -> DecodeCase:
    """Parallel sampling with copy-on-write.

    Each prompt's frames are shared by reference by all its branches.  Branch b has a
    private tail of T_b - 1 tokens (T_b ~ U{tail_lo..tail_hi}) that it shares with the
    parent it was forked from, so this step's token at position prompt_len + T_b - 1 lands
    in a shared frame whenever that position is not the first slot of a block: the frame is
    then copied to a fresh one (a copy pair), the branch's table is repointed, and the new
    token is written into the copy.  Otherwise the branch gets a fresh frame for it.
    """
    assert prompt_len % bs == 0
    src = "f32" if kv_dtype == "f32" else "bf16"
    rng = np.random.default_rng(seed)
    nbr = prompts * branches
    tails = rng.integers(tail_lo, tail_hi + 1, size=nbr).astype(np.int64)
    lens = prompt_len + tails
    pblk = prompt_len // bs
    tblk = -(-(tails - 1) // bs)
    NB = prompts * pblk + int(tblk.sum()) + nbr + spare
    perm = rng.permutation(NB)
    off = 0
    prompt_frames = perm[off : off + prompts * pblk].reshape(prompts, pblk)
    off += prompts * pblk
    tail_frames = []
    for b in range(nbr):
        tail_frames.append(perm[off : off + tblk[b]])
        off += int(tblk[b])
    fresh = perm[off : off + nbr]
    off += nbr
    width = int((-(-lens // bs)).max())
    tables = np.full((nbr, width), -1, dtype=np.int32)
    pairs = []
    for b in range(nbr):
        p = b // branches
        row = np.concatenate([prompt_frames[p], tail_frames[b]])
        tables[b, : len(row)] = row
        pos = int(lens[b]) - 1
        lb = pos // bs
        if pos % bs != 0:
            assert lb == len(row) - 1
            pairs.append((int(row[lb]), int(fresh[b])))
        else:
            assert lb == len(row)
        tables[b, lb] = fresh[b]
    q = _draw(rng, (nbr, Hq, D), std, src)
    pool_k = _draw(rng, (NB * bs, Hkv, D), std, src)
    pool_v = _draw(rng, (NB * bs, Hkv, D), std, src)
    new_k = _draw(rng, (nbr, Hkv, D), std, src)
    new_v = _draw(rng, (nbr, Hkv, D), std, src)
    live = np.zeros(NB * bs, dtype=bool)
    for p in range(prompts):
        f = prompt_frames[p].astype(np.int64)
        live[(f[:, None] * bs + np.arange(bs)[None, :]).ravel()] = True
    for b in range(nbr):
        f = tail_frames[b].astype(np.int64)
        pos = np.arange(int(tails[b]) - 1)
        live[f[pos // bs] * bs + pos % bs] = True
    new_slots = np.array([int(tables[b, (lens[b] - 1) // bs]) * bs + int((lens[b] - 1) % bs)
                          for b in range(nbr)], dtype=np.int64)
    _poison(pool_k, pool_v, live, src)
    ks, vs = (1.0, 1.0)
    if kv_dtype == "fp8":
        ks, vs = _fp8_scales(pool_k, pool_v, live, new_k, new_v, src)
    return DecodeCase(name=name, seed=seed, B=nbr, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
                      q_dtype=src, kv_dtype=kv_dtype, src_dtype=src,
                      scale=1.0 / math.sqrt(D), k_scale=ks, v_scale=vs,
                      context_lens=lens.astype(np.int32), block_tables=tables, q=q,
                      pool_k=pool_k, pool_v=pool_v, new_k=new_k, new_v=new_v,
                      new_slots=new_slots,
                      copy_pairs=np.array(pairs, dtype=np.int64).reshape(-1, 2),
                      meta={"live_slots": int(live.sum()), "prompt_frames": prompt_frames,
                            "tails": tails, "unique_frames": NB - spare})


def _loguniform_lens(lo: int, hi: int, n: int):
    def draw(rng):
        u = rng.uniform(math.log(lo), math.log(hi), size=n)
        return np.clip(np.round(np.exp(u)), lo, hi).astype(np.int64)
    return draw


def _uniform_lens(lo: int, hi: int, n: int):
    return lambda rng: rng.integers(lo, hi + 1, size=n).astype(np.int64)


def config5_variant(kv_dtype: str = "bf16", bs: int = 16, seed: int = 5) -> DecodeCase:
    """Config 5's mixed step (a 512-token chunk at 16,384 tokens + 128 decodes, Llama-3-8B
    shapes) with another KV dtype or block size: the fp8 / 32-token-block prefill variants."""
    c = chunk_case(f"llama3-8b-mixed chunk512@16384 + 128 decodes {kv_dtype} bs{bs}", seed, Hq=32,
                   Hkv=8, D=128, bs=bs, chunks=[(512, 16384)],
                   decode_lens=_uniform_lens(256, 4096, 128), kv_dtype=kv_dtype,
                   std=1.0 / math.sqrt(2.0))
    c.meta["cfg"] = 5
    return c


def long_context(n: int, L: int = 32768, seed: int | None = None) -> DecodeCase:
    """n sequences of L context tokens at the Llama-3-70B layer shape (64 query heads, 8 KV
    heads, head_dim 128, bf16, 16-token blocks, values N(0,1)/sqrt(2)) over a scattered pool:
    the long-context regime, a 32,000-token document as bicarait.com's "Architectural
    Blueprint 3" speaks of, where a few sequences' contexts are split across the whole GPU."""
    c = decode_case(f"llama3-70b-decode-long bf16 B{n} L{L} Hq64 Hkv8 D128 bs16",
                    600 + n if seed is None else seed, Hq=64, Hkv=8, D=128, bs=16, lens=[L] * n,
                    kv_dtype="bf16", std=1.0 / math.sqrt(2.0), pool="scattered")
    c.meta["cfg"] = "long"
    return c


def make(cfg: int, seed: int | None = None) -> DecodeCase:
    """The five named workloads at full size (seed defaults to the config number)."""
    seed = cfg if seed is None else seed
    s2 = 1.0 / math.sqrt(2.0)
    if cfg == 1:
        c = decode_case(CONFIG_NAMES[1], seed, Hq=4, Hkv=2, D=64, bs=16,
                        lens=[1, 17, 100, 255], kv_dtype="f32", std=1.0, pool=64)
    elif cfg == 2:
        c = decode_case(CONFIG_NAMES[2], seed, Hq=32, Hkv=8, D=128, bs=16,
                        lens=_uniform_lens(512, 4096, 64), kv_dtype="bf16", std=s2,
                        pool="exact")
    elif cfg == 3:
        c = decode_case(CONFIG_NAMES[3], seed, Hq=64, Hkv=8, D=128, bs=16,
                        lens=_loguniform_lens(128, 8192, 256), kv_dtype="bf16", std=s2,
                        pool="scattered")
    elif cfg == 4:
        c = fork_case(CONFIG_NAMES[4], seed)
    elif cfg == 5:
        c = chunk_case(CONFIG_NAMES[5], seed, Hq=32, Hkv=8, D=128, bs=16,
                       chunks=[(512, 16384)], decode_lens=_uniform_lens(256, 4096, 128),
                       kv_dtype="bf16", std=s2)
    else:
        raise ValueError(f"unknown config {cfg}")
    c.meta["cfg"] = cfg
    return c

# ----------------------------------------------------------------------------- steered scores

SCORE_PROFILES = ("rising", "spike", "falling")


def steer_scores(case: DecodeCase, seed: int, profile: str, span: float = 60.0) -> DecodeCase:
    """The same case with its attention scores steered along the context.

    Every query head of KV head g and every key of g lie near one unit direction u_g (queries
    a u_g, keys beta(t) u_g, each plus N(0, 0.05^2) per element), so a key's scaled score
    (scale * log2(e) * q.K, the softmax weight's log2) is set by a profile of its position t,
    the same for every sequence that holds the key (shared frames hold one position):
      rising   climbs by `span` from position 0 to the longest context's last position
      falling  falls by `span` over the same positions
      spike    a random level in [-2, 2], with one key `span` above it at 3/4 of the longest
               context and one span/2 above it at 1/3
    Tables, lengths, V, copy pairs and the poison in unwritten slots are unchanged; fp8
    scales are recomputed from the new keys.  Only inputs are built here.
    """
    if profile not in SCORE_PROFILES:
        raise ValueError(f"profile must be one of {SCORE_PROFILES}")
    c = case
    rng = np.random.default_rng(seed)
    src, D, bs = c.src_dtype, c.D, c.bs
    pos = np.full(c.NB * bs, -1, dtype=np.int64)
    seqs = [(c.block_tables[b], int(c.context_lens[b])) for b in range(c.B)]
    ch = c.chunk
    if ch is not None:
        seqs += [(ch.block_tables[i], int(ch.context_lens[i])) for i in range(ch.num_chunks)]
    for table, L in seqs:
        t = np.arange(L, dtype=np.int64)
        pos[_slots(table, t, bs)] = t
    for src_f, dst_f in c.copy_pairs:  # a copied frame holds the positions of its copy
        a = np.arange(bs, dtype=np.int64)
        s_sl, d_sl = src_f * bs + a, dst_f * bs + a
        keep = pos[s_sl] < 0
        pos[s_sl[keep]] = pos[d_sl[keep]]
    t_max = max(1, max(L for _, L in seqs) - 1)
    a_q = 4.0
    per_unit = c.scale * math.log2(math.e) * a_q  # scaled score of beta = 1
    tt = np.arange(t_max + 1, dtype=np.float64)
    if profile == "rising":
        target = span * tt / t_max
    elif profile == "falling":
        target = span * (1.0 - tt / t_max)
    else:
        target = rng.uniform(-2.0, 2.0, size=t_max + 1)
        target[(3 * t_max) // 4] += span
        target[t_max // 3] += span / 2.0
    beta = target / per_unit
    u = rng.standard_normal((c.Hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)

    def keys(p):  # p: positions [n] -> [n, Hkv, D] keys
        k = beta[p][:, None, None] * u[None] + 0.05 * rng.standard_normal((len(p), c.Hkv, D))
        return k.astype(np.float32)

    def enc(x, dtype):
        return x.astype(np.float32) if dtype == "f32" else _bf16_bits(x)

    def queries(n):
        g = np.arange(c.Hq) // c.G
        x = a_q * u[g][None] + 0.05 * rng.standard_normal((n, c.Hq, D))
        return x.astype(np.float32)

    pool_k = c.pool_k.copy()
    live = pos >= 0  # slots holding a key before the step (the step's new slots hold poison)
    live[c.new_slots] = False
    pool_k[live] = enc(keys(pos[live]), src)
    new_pos = pos[c.new_slots]
    assert (new_pos >= 0).all(), "every new row sits at a position of some sequence"
    new_k = enc(keys(new_pos), src)
    q = enc(queries(c.B), c.q_dtype) if c.B else c.q
    chunk = ch
    if ch is not None:
        chunk = ChunkPart(q=enc(queries(ch.q.shape[0]), c.q_dtype),
                          query_start_loc=ch.query_start_loc, context_lens=ch.context_lens,
                          block_tables=ch.block_tables, new_rows=ch.new_rows)
    ks, vs = c.k_scale, c.v_scale
    if c.kv_dtype == "fp8":
        ks, vs = _fp8_scales(pool_k, c.pool_v, live, new_k, c.new_v, src)
    return replace(c, q=q, pool_k=pool_k, new_k=new_k, chunk=chunk, k_scale=ks, v_scale=vs,
                   meta=dict(c.meta, profile=profile))
