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
