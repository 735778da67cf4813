"""The block manager driving the GPU path: prompts, forks into sampling branches, decode steps
with copy-on-write, release and reuse of frames.  The library's C++ manager feeds the kernels
(pa_copy_blocks, pa_reshape_and_cache, pa_decode); the reference model feeds the oracle.  At
every step the block tables must agree, the caches must be bit-identical and the decode outputs
within tolerance of the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_256_amd as pa
from oracle import BlockManagerModel
from tests.gpu_harness import device, out_f64, to_dev, to_raw

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, NB = 8, 2, 128, 16, 96
SCALE = 1.0 / np.sqrt(D)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_block_manager_drives_decode(kv):
    print(f"block manager scenario, kv {kv}", flush=True)
    rng = np.random.default_rng(21)
    dev = device()
    bm, model = pa.BlockManager(NB, BS), BlockManagerModel(NB, BS)
    kc, vc = pa.new_kv_cache(NB, HKV, BS, D, kv, device=dev)
    kc.zero_()                                # frames never written compare equal to the
    vc.zero_()                                # oracle's zero-initialised caches
    okc, ovc = oracle.new_cache(NB, HKV, BS, D, kv), oracle.new_cache(NB, HKV, BS, D, kv)
    k_scale = v_scale = 3.0 / 448 if kv == "fp8" else 1.0
    kw = dict(bs=BS, src_dtype="bf16", kv_dtype=kv, k_scale=k_scale, v_scale=v_scale)

    def step(ids):
        slots, copies = bm.append(ids)
        want_slots, want_copies = model.append(ids)
        assert list(slots) == want_slots and [tuple(c) for c in copies] == want_copies
        n = len(ids)
        k = _bf16_bits(rng.standard_normal((n, HKV, D)) * 0.7071)
        v = _bf16_bits(rng.standard_normal((n, HKV, D)) * 0.7071)
        if len(copies):
            pa.copy_blocks(kc, vc, to_dev(copies.astype(np.int64), "i64", dev), block_size=BS, kv_dtype=kv)
            oracle.copy_blocks(okc, ovc, copies)
        pa.reshape_and_cache(to_dev(k, "bf16", dev), to_dev(v, "bf16", dev), kc, vc,
                             to_dev(slots, "i64", dev), block_size=BS, kv_dtype=kv,
                             k_scale=k_scale, v_scale=v_scale)
        oracle.reshape_and_cache(okc, ovc, k, v, slots, **kw)

    def decode(seqs):
        width = max(len(model.tables[s]) for s in seqs)
        tables, lens = bm.block_tables(seqs, width)
        for i, s in enumerate(seqs):
            t, L = model.block_table(s, width)
            assert list(tables[i]) == t and lens[i] == L
        q = _bf16_bits(rng.standard_normal((len(seqs), HQ, D)) * 0.7071)
        out = pa.decode(to_dev(q, "bf16", dev), kc, vc, to_dev(tables, "i32", dev),
                        to_dev(lens, "i32", dev), block_size=BS, scale=SCALE, kv_dtype=kv,
                        max_context_len=int(lens.max()), k_scale=k_scale, v_scale=v_scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_raw(kc), okc)
        np.testing.assert_array_equal(to_raw(vc), ovc)
        want = oracle.decode(q, okc, ovc, tables, lens, scale=SCALE, bs=BS, q_dtype="bf16",
                             kv_dtype=kv, k_scale=k_scale, v_scale=v_scale)
        err = np.abs(out_f64(out) - want).max()
        assert err <= 1e-2, err

    step([0] * 70 + [1] * 20)                 # two prompts (70 tokens: a partly filled frame)
    for b in (2, 3, 4):
        bm.fork(0, b)
        model.fork(0, b)                      # three sampling branches of prompt 0
    for _ in range(3):                        # decode steps: the first writes copy frame 4
        step([0, 1, 2, 3, 4])
        decode([0, 1, 2, 3, 4])
    bm.free(1)
    model.release(1)                          # a finished sequence returns its frames
    step([5] * 33)                            # a new prompt reuses them
    for _ in range(2):
        step([0, 2, 3, 4, 5])
        decode([0, 2, 3, 4, 5])
    assert bm.num_free() == len(model.free)
    bm.close()


def _kv_rows(tokens, positions):
    """K and V rows (bf16 bits) that depend only on (token id, position): a prefix computed once
    is exactly what recomputing it would give."""
    k = np.empty((len(tokens), HKV, D), np.float32)
    v = np.empty((len(tokens), HKV, D), np.float32)
    for i, (t, p) in enumerate(zip(tokens, positions)):
        r = np.random.default_rng(int(t) * 100003 + int(p))
        k[i] = r.standard_normal((HKV, D)) * 0.7071
        v[i] = r.standard_normal((HKV, D)) * 0.7071
    return _bf16_bits(k), _bf16_bits(v)


def test_prefix_cached_prompts_decode_exactly():
    print("prefix caching scenario", flush=True)
    rng = np.random.default_rng(33)
    dev = device()
    bm, model = pa.BlockManager(NB, BS), BlockManagerModel(NB, BS)
    kc, vc = pa.new_kv_cache(NB, HKV, BS, D, "bf16", device=dev)
    kc.zero_()
    vc.zero_()
    okc, ovc = oracle.new_cache(NB, HKV, BS, D, "bf16"), oracle.new_cache(NB, HKV, BS, D, "bf16")
    kw = dict(bs=BS, src_dtype="bf16", kv_dtype="bf16")
    history = {}

    def write(slots, toks, pos):
        if not len(slots):
            return
        k, v = _kv_rows(toks, pos)
        pa.reshape_and_cache(to_dev(k, "bf16", dev), to_dev(v, "bf16", dev), kc, vc,
                             to_dev(np.asarray(slots, np.int64), "i64", dev), block_size=BS,
                             kv_dtype="bf16")
        oracle.reshape_and_cache(okc, ovc, k, v, np.asarray(slots, np.int64), **kw)

    def prompt(seq, toks):
        slots, cached = bm.append_prompt(seq, toks)
        want_slots, want_cached = model.append_prompt(seq, toks)
        assert list(slots) == want_slots and cached == want_cached
        # only the tokens the prefix tree did not supply are computed and written
        write(slots[cached:], toks[cached:], list(range(cached, len(toks))))
        history[seq] = list(toks)
        return cached

    def decode_step(seqs):
        new = [int(t) for t in rng.integers(0, 1000, size=len(seqs))]
        slots, copies = bm.append(seqs)
        want_slots, want_copies = model.append(seqs)
        assert list(slots) == want_slots and [tuple(c) for c in copies] == want_copies
        assert not len(copies)
        write(slots, new, [len(history[s]) for s in seqs])
        for s, t in zip(seqs, new):
            history[s].append(t)
        width = max(len(model.tables[s]) for s in seqs)
        tables, lens = bm.block_tables(seqs, width)
        q = _bf16_bits(rng.standard_normal((len(seqs), HQ, D)) * 0.7071)
        out = pa.decode(to_dev(q, "bf16", dev), kc, vc, to_dev(tables, "i32", dev),
                        to_dev(lens, "i32", dev), block_size=BS, scale=SCALE, kv_dtype="bf16",
                        max_context_len=int(lens.max()))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_raw(kc), okc)
        np.testing.assert_array_equal(to_raw(vc), ovc)
        # every sequence's context, read through its table, is its own tokens' K/V
        for i, s in enumerate(seqs):
            kg = oracle.gather_kv(okc, tables[i], int(lens[i]), "k", bs=BS, kv_dtype="bf16")
            vg = oracle.gather_kv(ovc, tables[i], int(lens[i]), "v", bs=BS, kv_dtype="bf16")
            kw_, vw_ = _kv_rows(history[s], range(len(history[s])))
            np.testing.assert_array_equal(kg, oracle.bf16_bits_to_f64(kw_))
            np.testing.assert_array_equal(vg, oracle.bf16_bits_to_f64(vw_))
        want = oracle.decode(q, okc, ovc, tables, lens, scale=SCALE, bs=BS, q_dtype="bf16",
                             kv_dtype="bf16")
        assert np.abs(out_f64(out) - want).max() <= 1e-2

    system = [int(t) for t in rng.integers(0, 1000, size=40)]       # 2 full blocks + 8 tokens
    assert prompt(0, system + [1, 2, 3]) == 0
    assert prompt(1, system + [4, 5, 6, 7, 8, 9, 10]) == 32         # two blocks reused
    decode_step([0, 1])
    bm.free(0)
    model.release(0)
    assert prompt(2, system + list(range(20))) == 32                # revived after release
    decode_step([1, 2])
    decode_step([1, 2])
    bm.close()
