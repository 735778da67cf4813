"""GPU parity of pa_mixed_attention: the decodes and prefill chunks of a step in one persistent
kernel, against the fp64 oracle (decode rows within the decode tolerance, chunk rows within the
chunk tolerance; caches bit-exact).  The launch's split of compute units between the two halves
follows the caller's decode-token count: results must hold for any split and be bit-identical
for a repeated call."""

import numpy as np
import pytest
import torch

import paged_kv_cache_256_amd as pa
import workloads
from tests.gpu_harness import GpuStep, OracleStep, out_f64, to_raw, tolerance

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(g, o, dec, chunk, decode_seqs=None, chunk_rows=None):
    c = g.c
    tol = tolerance(c)
    errs = []
    if c.B:
        seqs = list(range(c.B)) if decode_seqs is None else list(decode_seqs)
        got = out_f64(dec)[seqs]
        assert np.isfinite(got).all()
        errs.append(np.abs(got - o.decode(seqs)).max())
    if c.chunk is not None and c.chunk.num_chunks:
        got = out_f64(chunk)
        assert np.isfinite(got).all()
        want = o.prefill(chunk_rows)
        if chunk_rows is not None:
            got, want = got[chunk_rows], want[chunk_rows]
        errs.append(np.abs(got - want).max())
    err = max(errs)
    assert err <= tol, f"max abs err {err:.3e} > {tol}"
    return err


MIXED_CASES = [
    # kv, D, bs, G, chunks (C, L), decode lengths
    ("f32", 64, 16, 2, [(20, 70), (16, 16), (37, 100)], [5, 33, 200]),
    ("f32", 128, 16, 1, [(40, 300)], [1, 513]),
    ("bf16", 128, 16, 4, [(512, 2048)], [100, 1, 3000, 17]),
    ("bf16", 128, 32, 8, [(100, 300), (64, 64)], [40, 1025]),
    ("bf16", 64, 16, 16, [(33, 33), (70, 500)], [20]),
    ("bf16", 64, 32, 2, [(90, 700)], [64, 65, 2000]),
    ("bf16", 128, 16, 1, [(130, 900)], [900, 1]),
    ("fp8", 128, 32, 4, [(200, 1000)], [77, 2500]),
    ("fp8", 64, 16, 8, [(64, 600)], [5, 600, 33]),
    ("bf16", 128, 16, 4, [(300, 1200)], []),
    ("bf16", 128, 16, 4, [], [100, 2000, 7]),
]


@pytest.mark.parametrize("mode", ["split", "separate"])
@pytest.mark.parametrize("kv,D,bs,G,chunks,dec", MIXED_CASES,
                         ids=[f"{c[0]}-D{c[1]}-bs{c[2]}-G{c[3]}-{len(c[4])}ch-{len(c[5])}dec"
                              for c in MIXED_CASES])
def test_mixed_small(kv, D, bs, G, chunks, dec, mode):
    Hkv = 2
    _say(f"mixed case kv={kv} D={D} bs={bs} G={G} chunks={chunks} decodes={dec} mode={mode}")
    c = workloads.chunk_case("mixed", 300 + D + G + bs, Hq=G * Hkv, Hkv=Hkv, D=D, bs=bs,
                             chunks=chunks, decode_lens=dec, kv_dtype=kv,
                             std=1.0 if kv == "f32" else 0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.write()
    d, ch = g.mixed(mode=mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    np.testing.assert_array_equal(to_raw(g.vc), o.vc)
    err = _check(g, o, d, ch)
    _say(f"  max abs err {err:.2e}")


def test_mixed_every_mode_and_hint_is_correct_and_repeat_is_bit_identical():
    c = workloads.chunk_case("mixed-split", 41, Hq=16, Hkv=4, D=128, bs=16,
                             chunks=[(256, 1500), (100, 100)],
                             decode_lens=[1, 16, 17, 400, 1200, 3000, 64, 900], kv_dtype="bf16",
                             std=0.7071)
    m = workloads.mixed_batch(c)
    g, o = GpuStep(c), OracleStep(c)
    g.write()
    units = set()
    for mode in ("auto", "split", "separate"):
        for hint in (m.decode_tokens, 1, 10 ** 12):
            P = pa.mixed_prefill_units(m.num_decodes, c.chunk.num_chunks, m.q.shape[0],
                                       m.max_chunk_len, m.max_context_len, hint, c.Hq, c.Hkv, c.D,
                                       c.bs, c.kv_dtype, mode)
            _say(f"mode {mode}, decode_tokens hint {hint}: {P} prefill workgroups")
            units.add(P)
            d, ch = g.mixed(decode_tokens=hint, mode=mode)
            first = (d.clone(), ch.clone())
            d2, ch2 = g.mixed(decode_tokens=hint, mode=mode)
            torch.cuda.synchronize()
            assert torch.equal(first[0], d2) and torch.equal(first[1], ch2)
            _check(g, o, first[0], first[1])
    assert len(units) >= 3, f"modes and hints should give different launches, got {units}"


@pytest.mark.parametrize("mode", ["split", "separate"])
def test_mixed_plan_kernel_path_above_1024_decodes(mode):
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 300, size=1100)
    c = workloads.chunk_case("mixed-big", 43, Hq=8, Hkv=2, D=64, bs=16, chunks=[(256, 1024)],
                             decode_lens=lens, kv_dtype="bf16", std=0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.write()
    d, ch = g.mixed(mode=mode)
    torch.cuda.synchronize()
    err = _check(g, o, d, ch)
    _say(f"  1100 decodes + chunk ({mode}): max abs err {err:.2e}")


def test_mixed_matches_separate_calls_within_tolerance():
    c = workloads.chunk_case("mixed-vs-sep", 44, Hq=32, Hkv=8, D=128, bs=16,
                             chunks=[(512, 4096)], decode_lens=[50, 700, 2048, 4000] * 4,
                             kv_dtype="bf16", std=0.7071)
    g = GpuStep(c)
    g.write()
    d, ch = g.mixed()
    sd = g.decode()
    sc = g.prefill()
    torch.cuda.synchronize()
    assert (out_f64(d) - out_f64(sd)).__abs__().max() <= 2 * tolerance(c)
    assert (out_f64(ch) - out_f64(sc)).__abs__().max() <= 2 * tolerance(c)
