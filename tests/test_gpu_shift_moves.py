"""GPU parity when the softmax's running shift has to move.

The decode and prefill kernels move their running shift lazily: only when a step's scaled
scores exceed it by more than 2^8 are the accumulators rescaled.  With normal random inputs a
shift set on the first step is rarely exceeded later, so these cases steer the scores along
the context (workloads.steer_scores): scores that climb by 60 log2 units (the shift moves at
many steps, and the pieces of a run cut across wavefronts carry different shifts into the
merge), a late spike 60 units above everything before it, and scores that fall from the first
key.  Every output is compared with the fp64 oracle, as in the other parity tests.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_256_amd as pa
import workloads
from tests.gpu_harness import GpuStep, OracleStep, out_f64, to_raw, tolerance

pytestmark = pytest.mark.gpu

PROFILES = workloads.SCORE_PROFILES


def _say(msg):
    print(msg, flush=True)


def _tol(c) -> float:
    """The parity bound of these cases.  bf16 / fp8: the usual 1e-2.  f32: the logits here are
    large (scaled scores up to S = 60 log2 units, raw q.K up to S / (scale log2 e)), and an fp32
    score's rounding error grows with them: about S sqrt(D) 2^-24 ~ 3e-5 in log2 units for
    D = 64, a relative weight error of ~2e-5, up to ~1e-4 on outputs with |V| up to ~4.5.  The
    usual f32 bound of 1e-5 is set for unit-scale logits; a wrong rescale is off by O(1)."""
    return 1e-4 if c.kv_dtype == "f32" else tolerance(c)


def _err(got, want, c):
    got = out_f64(got) if isinstance(got, torch.Tensor) else got
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= _tol(c), f"max abs err {err:.3e} > {_tol(c)}"
    return err


DECODE = [
    # kv, D, bs, G, lengths
    ("f32", 64, 16, 4, [1, 33, 700, 2100]),
    ("bf16", 128, 16, 8, [1, 33, 700, 2100, 4100]),
    ("fp8", 128, 32, 8, [1, 40, 1000, 3000]),
]


@pytest.mark.parametrize("profile", PROFILES)
@pytest.mark.parametrize("kv,D,bs,G,lens", DECODE, ids=[f"{d[0]}-D{d[1]}-bs{d[2]}-G{d[3]}" for d in DECODE])
def test_decode_with_moving_shift(kv, D, bs, G, lens, profile):
    _say(f"decode kv={kv} D={D} bs={bs} G={G} lens={lens} profile={profile}")
    base = workloads.decode_case("shift", 900 + D + bs, Hq=2 * G, Hkv=2, D=D, bs=bs, lens=lens,
                                 kv_dtype=kv, std=1.0 if kv == "f32" else 0.7071, pool="scattered")
    c = workloads.steer_scores(base, 31, profile)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    err = _err(g.out, o.decode(), c)
    _say(f"  max abs err {err:.2e}")


PREFILL = [
    # kv, D, bs, G, chunks (C, L)
    ("f32", 64, 16, 2, [(40, 1200), (16, 16)]),
    ("bf16", 128, 16, 4, [(64, 3000), (130, 130), (17, 1500)]),
    ("fp8", 128, 32, 4, [(200, 2600)]),
]


@pytest.mark.parametrize("profile", PROFILES)
@pytest.mark.parametrize("kv,D,bs,G,chunks", PREFILL, ids=[f"{d[0]}-D{d[1]}-bs{d[2]}-G{d[3]}" for d in PREFILL])
def test_prefill_with_moving_shift(kv, D, bs, G, chunks, profile):
    _say(f"prefill kv={kv} D={D} bs={bs} G={G} chunks={chunks} profile={profile}")
    base = workloads.chunk_case("shift-chunk", 950 + D + bs, Hq=2 * G, Hkv=2, D=D, bs=bs,
                                chunks=chunks, decode_lens=[3, 900], kv_dtype=kv,
                                std=1.0 if kv == "f32" else 0.7071)
    c = workloads.steer_scores(base, 37, profile)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    err = _err(g.chunk_out, o.prefill(), c)
    err = max(err, _err(g.out, o.decode(), c))
    # the single-launch mixed batch over the same step (its own split of the work)
    for mode in ("split", "separate"):
        dec, rows = g.mixed(mode=mode)
        torch.cuda.synchronize()
        err = max(err, _err(dec, o.decode(), c), _err(rows, o.prefill(), c))
    _say(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("profile", PROFILES)
def test_shared_decode_with_moving_shift(profile):
    """pa_decode_shared: each run's members keep their own shift per score column."""
    base = workloads.fork_case("shift-shared", 977, prompts=3, branches=6, prompt_len=1024,
                               tail_lo=1, tail_hi=900, Hq=16, Hkv=2, D=128, bs=32,
                               kv_dtype="fp8", std=0.7071)
    c = workloads.steer_scores(base, 41, profile)
    _say(f"shared decode, profile={profile}")
    runs = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs,
                                   pa.SHARED_RUN_COLUMNS // (c.Hq // c.Hkv))
    g = GpuStep(c)
    g.write()
    out = pa.decode_shared(g.q, g.kc, g.vc, g.tables, g.lens, runs.to(g.dev), block_size=c.bs,
                           scale=c.scale, kv_dtype=c.kv_dtype, max_context_len=c.max_context_len,
                           k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    o = OracleStep(c)
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    err = _err(out, o.decode(), c)
    _say(f"  {runs.num_runs} runs: max abs err {err:.2e}")
