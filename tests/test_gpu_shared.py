"""GPU parity of pa_decode_shared: decode of batches in which runs of consecutive sequences share
the first frames of their block tables (branches of one prompt), each run streaming its shared
frames once for all its members.  Every output is compared with the fp64 oracle's plain decode;
caches are bit-exact; a repeated call gives identical bits; and the result agrees with
pa_decode's."""

import numpy as np
import pytest
import torch

import paged_kv_cache_256_amd as pa
import workloads
from tests.gpu_harness import GpuStep, OracleStep, out_f64, to_raw, tolerance

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run_shared(g: GpuStep, runs):
    c = g.c
    return pa.decode_shared(g.q, g.kc, g.vc, g.tables, g.lens, runs.to(g.dev), block_size=c.bs,
                            scale=c.scale, kv_dtype=c.kv_dtype, max_context_len=c.max_context_len,
                            k_scale=c.k_scale, v_scale=c.v_scale)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check(c, g, runs):
    pa.validate_shared_prefixes(c.block_tables, c.context_lens, c.bs, runs, c.Hq // c.Hkv)
    out1 = _run_shared(g, runs)
    out2 = _run_shared(g, runs)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out1), _bits(out2)), "repeated calls differ"
    o = OracleStep(c)
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    np.testing.assert_array_equal(to_raw(g.vc), o.vc)
    got = out_f64(out1)
    assert np.isfinite(got).all()
    err = np.abs(got - o.decode()).max()
    assert err <= tolerance(c), f"max abs err {err:.3e}"
    ref = out_f64(g.decode())
    torch.cuda.synchronize()
    assert np.abs(got - ref).max() <= 2 * tolerance(c)
    return err


def test_config4_every_output():
    c = workloads.make(4)
    runs = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs,
                                   pa.SHARED_RUN_COLUMNS // (c.Hq // c.Hkv))
    assert runs.num_runs == 128 and set(runs.run_size.tolist()) == {0, 2}
    g = GpuStep(c)
    g.write()
    err = _check(c, g, runs)
    _say(f"config 4: {runs.num_runs} runs of 2, max abs err {err:.2e} over all {c.B} sequences")


FORK_CASES = [
    # kv, D, bs, Hq, Hkv, prompts, branches, prompt_len, tails, max run
    ("fp8", 128, 32, 64, 8, 5, 8, 1024, (64, 512), 2),
    ("bf16", 128, 16, 64, 8, 4, 7, 640, (1, 300), 2),       # runs of 2, 2, 2 and one alone
    ("bf16", 128, 32, 32, 8, 3, 16, 512, (1, 100), 4),      # G 4: runs of 4
    ("bf16", 64, 16, 32, 2, 2, 6, 256, (2, 40), 1),         # G 16: every run alone (plain)
    ("bf16", 128, 16, 8, 8, 3, 40, 160, (1, 64), 16),       # G 1: runs of 16, 16 and 8
    ("fp8", 64, 16, 16, 4, 3, 5, 96, (1, 33), 3),           # G 4, runs of 3 and 2
    ("f32", 64, 16, 8, 4, 3, 7, 128, (1, 50), 8),           # f32, G 2
    ("f32", 128, 16, 4, 2, 2, 9, 64, (5, 20), 8),
    ("bf16", 128, 16, 64, 8, 1, 3, 32768, (1, 2000), 2),    # a long shared prefix, cut across ranges
]


@pytest.mark.parametrize("kv,D,bs,Hq,Hkv,P,Br,pl,tails,mr", FORK_CASES,
                         ids=[f"{c[0]}-D{c[1]}-bs{c[2]}-G{c[3] // c[4]}-{c[5]}x{c[6]}-r{c[9]}" for c in FORK_CASES])
def test_shared_prefix_runs(kv, D, bs, Hq, Hkv, P, Br, pl, tails, mr):
    _say(f"shared case kv={kv} D={D} bs={bs} G={Hq // Hkv} {P} prompts x {Br} branches, "
         f"prompt {pl}, runs of at most {mr}")
    c = workloads.fork_case("shared", 700 + D + bs + Br, prompts=P, branches=Br, prompt_len=pl,
                            tail_lo=tails[0], tail_hi=tails[1], Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                            kv_dtype=kv, std=1.0 if kv == "f32" else 0.7071)
    runs = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs, mr)
    g = GpuStep(c)
    g.write()
    err = _check(c, g, runs)
    _say(f"  {runs.num_runs} shared runs: max abs err {err:.2e}")


@pytest.mark.parametrize("prompts,branches", [(75, 8), (128, 8), (97, 7)],
                         ids=["600-seqs", "1024-seqs", "679-seqs"])
def test_shared_prefix_runs_in_wide_plan_blocks(prompts, branches):
    """Batches of 513-1,024 sequences planned inside the wavefronts: a plan lane then holds
    ceil(B / 64) = 9-16 sequences, and the runs are laid out head by head within those blocks,
    with prompts that straddle the blocks (7 branches per prompt)."""
    c = workloads.fork_case("shared-wide", 711 + prompts, prompts=prompts, branches=branches,
                            prompt_len=64, tail_lo=1, tail_hi=40, Hq=16, Hkv=2, D=64, bs=16,
                            kv_dtype="fp8", std=0.7071)
    assert 512 < c.B <= 1024
    runs = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs, 2)
    g = GpuStep(c)
    g.write()
    err = _check(c, g, runs)
    _say(f"{c.B} sequences, {runs.num_runs} runs: max abs err {err:.2e}")


def test_shared_prefix_runs_above_1024_sequences():
    """1,040 sequences (130 prompts x 8 branches): the ranges are planned by the one-workgroup
    plan kernel."""
    c = workloads.fork_case("shared-big", 709, prompts=130, branches=8, prompt_len=64, tail_lo=1,
                            tail_hi=40, Hq=16, Hkv=2, D=64, bs=16, kv_dtype="bf16", std=0.7071)
    runs = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs, 2)
    assert runs.num_runs == 520
    g = GpuStep(c)
    g.write()
    err = _check(c, g, runs)
    _say(f"1040 sequences: max abs err {err:.2e}")


def test_runs_of_one_are_plain_decodes():
    """Every sequence a run of its own (nothing shared) on the 70B-shape batch of 256: the same
    arithmetic as pa_decode, over the grouped launch's own split of the work (4 wavefronts per
    CU, so other cut points and merge orders: equal within rounding, not bit for bit)."""
    c = workloads.make(3)
    g = GpuStep(c)
    g.write()
    runs = pa.SharedRuns(np.zeros(c.B, np.int32), np.ones(c.B, np.int32))
    err = _check(c, g, runs)
    _say(f"config 3 as runs of one: max abs err {err:.2e}")
