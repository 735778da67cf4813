"""Runs one paged-attention step of a workload case on the GPU and on the CPU oracle.

Both sides start from the same seeded host arrays (workloads/).  The GPU side fills its
caches with pa_reshape_and_cache over every pool slot, applies the step's copy-on-write
pairs, writes the step's new K/V rows, then runs pa_prefill_chunk and pa_decode.  The
oracle side does the same with oracle/ on host arrays.  Nothing flows from the GPU into
the oracle.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_cache_256_amd as pa
import workloads


def device():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, kind: str, dev):
    """Host raw array (float32, bf16 bits as uint16, int32/int64) -> device tensor."""
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_raw(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host raw array (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


class GpuStep:
    """Device state of a case: caches after the initial fill, and the step's outputs."""

    def __init__(self, case, dev=None):
        self.c = c = case
        self.dev = dev = dev or device()
        s = c.src_dtype
        self.kc, self.vc = pa.new_kv_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype, device=dev)
        pk, pv = to_dev(c.pool_k, s, dev), to_dev(c.pool_v, s, dev)
        slots = torch.arange(c.NB * c.bs, dtype=torch.int64, device=dev)
        pa.reshape_and_cache(pk, pv, self.kc, self.vc, slots, block_size=c.bs, kv_dtype=c.kv_dtype,
                             k_scale=c.k_scale, v_scale=c.v_scale)
        del pk, pv, slots
        self.q = to_dev(c.q, c.q_dtype, dev)
        self.tables = to_dev(c.block_tables, "i32", dev)
        self.lens = to_dev(c.context_lens, "i32", dev)
        self.new_k = to_dev(c.new_k, s, dev)
        self.new_v = to_dev(c.new_v, s, dev)
        self.new_slots = to_dev(c.new_slots, "i64", dev)
        self.pairs = to_dev(c.copy_pairs, "i64", dev) if len(c.copy_pairs) else None
        if c.chunk is not None:
            ch = c.chunk
            self.cq = to_dev(ch.q, c.q_dtype, dev)
            self.ctables = to_dev(ch.block_tables, "i32", dev)
            self.cqsl = to_dev(ch.query_start_loc, "i32", dev)
            self.clens = to_dev(ch.context_lens, "i32", dev)
        self.out = None
        self.chunk_out = None

    def write(self):
        c = self.c
        if self.pairs is not None:
            pa.copy_blocks(self.kc, self.vc, self.pairs, block_size=c.bs, kv_dtype=c.kv_dtype)
        pa.reshape_and_cache(self.new_k, self.new_v, self.kc, self.vc, self.new_slots,
                             block_size=c.bs, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                             v_scale=c.v_scale)

    def prefill(self):
        c, ch = self.c, self.c.chunk
        self.chunk_out = pa.prefill_chunk(self.cq, self.kc, self.vc, self.ctables, self.cqsl,
                                          self.clens, block_size=c.bs, scale=c.scale,
                                          kv_dtype=c.kv_dtype, max_chunk_len=ch.max_chunk_len,
                                          max_context_len=ch.max_context_len, k_scale=c.k_scale,
                                          v_scale=c.v_scale)
        return self.chunk_out

    def decode(self, **kw):
        c = self.c
        self.out = pa.decode(self.q, self.kc, self.vc, self.tables, self.lens, block_size=c.bs,
                             scale=c.scale, kv_dtype=c.kv_dtype,
                             max_context_len=kw.pop("max_context_len", c.max_context_len),
                             k_scale=c.k_scale, v_scale=c.v_scale,
                             shared_frames=kw.pop("shared_frames", c.shares_frames), **kw)
        return self.out

    def mixed(self, decode_tokens=None, **kw):
        """pa_mixed_attention over the case's decodes and chunks as one batch (decodes first);
        returns the output split into (decode rows, chunk rows)."""
        c, dev = self.c, self.dev
        m = workloads.mixed_batch(c)
        if not hasattr(self, "_mixed_in"):
            self._mixed_in = (to_dev(m.q, c.q_dtype, dev), to_dev(m.block_tables, "i32", dev),
                              to_dev(m.query_start_loc, "i32", dev),
                              to_dev(m.context_lens, "i32", dev))
        q, tables, qsl, lens = self._mixed_in
        out = pa.mixed_attention(q, self.kc, self.vc, tables, qsl, lens, m.num_decodes,
                                 block_size=c.bs, scale=c.scale, kv_dtype=c.kv_dtype,
                                 max_chunk_len=max(m.max_chunk_len, 1),
                                 max_context_len=m.max_context_len,
                                 decode_tokens=m.decode_tokens if decode_tokens is None else decode_tokens,
                                 k_scale=c.k_scale, v_scale=c.v_scale,
                                 shared_frames=kw.pop("shared_frames", c.shares_frames),
                                 mode=kw.pop("mode", "auto"), **kw)
        self.mixed_out = out
        return out[:c.B], out[c.B:]

    def step(self):
        self.write()
        if self.c.chunk is not None:
            self.prefill()
        if self.c.B:
            self.decode()
        torch.cuda.synchronize(self.dev)


class OracleStep:
    """Host caches after the initial fill, the copies and the step's writes."""

    def __init__(self, case):
        self.c = c = case
        kw = dict(bs=c.bs, src_dtype=c.src_dtype, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                  v_scale=c.v_scale)
        self.kc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype)
        self.vc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype)
        oracle.reshape_and_cache(self.kc, self.vc, c.pool_k, c.pool_v, c.pool_slots, batch=8192, **kw)
        if len(c.copy_pairs):
            oracle.copy_blocks(self.kc, self.vc, c.copy_pairs)
        oracle.reshape_and_cache(self.kc, self.vc, c.new_k, c.new_v, c.new_slots, **kw)

    def decode(self, seqs=None):
        c = self.c
        return oracle.decode(c.q, self.kc, self.vc, c.block_tables, c.context_lens, scale=c.scale,
                             bs=c.bs, q_dtype=c.q_dtype, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                             v_scale=c.v_scale, seqs=seqs)

    def prefill(self, rows=None):
        c, ch = self.c, self.c.chunk
        return oracle.prefill_chunk(ch.q, self.kc, self.vc, ch.block_tables, ch.query_start_loc,
                                    ch.context_lens, scale=c.scale, bs=c.bs, q_dtype=c.q_dtype,
                                    kv_dtype=c.kv_dtype, k_scale=c.k_scale, v_scale=c.v_scale,
                                    rows=rows)


def tolerance(case) -> float:
    """max-abs bound against the oracle: 1e-5 for f32 outputs, 1e-2 for bf16 (bf16 or fp8 KV)."""
    return 1e-5 if case.kv_dtype == "f32" else 1e-2
