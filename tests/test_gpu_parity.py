"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Cache writes and block copies must match bit for bit over the whole pool; attention outputs
must be within 1e-5 (f32) or 1e-2 (bf16 / fp8 KV) max-abs of the fp64 oracle.  Sizes here are
small enough for the oracle to check every output and still span several partitions, splits
and ragged tails; tests/test_gpu_configs.py covers the five named workloads at full size.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_256_amd as pa
import workloads
from tests.gpu_harness import GpuStep, OracleStep, device, out_f64, to_dev, to_raw, tolerance

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_caches(g: GpuStep, o: OracleStep):
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    np.testing.assert_array_equal(to_raw(g.vc), o.vc)


def _check_decode(g: GpuStep, o: OracleStep, seqs=None):
    seqs = list(range(g.c.B)) if seqs is None else list(seqs)
    want = o.decode(seqs)
    got = out_f64(g.out)[seqs]
    err = np.abs(got - want).max()
    assert np.isfinite(got).all()
    assert err <= tolerance(g.c), f"max abs err {err:.3e} > {tolerance(g.c)}"
    return err


DECODE_CASES = [
    # kv dtype, D, bs, G, lengths
    ("f32", 64, 16, 2, [1, 17, 100, 255]),
    ("f32", 64, 32, 4, [1, 31, 32, 33, 700]),
    ("f32", 128, 16, 1, [5, 513, 1030]),
    ("bf16", 128, 16, 8, [1, 2, 15, 16, 17, 511, 512, 513, 1500, 3000]),
    ("bf16", 64, 16, 4, [3, 600, 1025]),
    ("bf16", 128, 32, 16, [40, 1024, 1025, 2100]),
    ("bf16", 64, 32, 2, [64, 65, 2000]),
    ("fp8", 128, 32, 8, [1, 33, 1023, 1024, 1025, 2500]),
    ("fp8", 64, 16, 4, [7, 512, 513, 900]),
    ("fp8", 128, 16, 1, [300, 1100]),
]


@pytest.mark.parametrize("kv,D,bs,G,lens", DECODE_CASES,
                         ids=[f"{c[0]}-D{c[1]}-bs{c[2]}-G{c[3]}" for c in DECODE_CASES])
def test_decode_small(kv, D, bs, G, lens):
    Hkv = 2
    _say(f"decode case kv={kv} D={D} bs={bs} G={G} lens={lens}")
    c = workloads.decode_case("small", 100 + D + bs + G, Hq=G * Hkv, Hkv=Hkv, D=D, bs=bs,
                              lens=lens, kv_dtype=kv, std=1.0 if kv == "f32" else 0.7071,
                              pool="scattered")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    _check_decode(g, o)


def test_config1_tiny_f32():
    c = workloads.make(1)
    _say("config 1")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    err = _check_decode(g, o)
    _say(f"config 1 max abs err {err:.2e}")


CHUNK_CASES = [
    # kv, D, bs, G, chunks (C, L), decode lengths
    ("f32", 64, 16, 2, [(20, 70), (16, 16), (37, 100)], [5, 33]),
    ("bf16", 128, 16, 4, [(512, 2048)], [100]),
    ("bf16", 128, 32, 8, [(100, 300), (64, 64)], []),
    ("bf16", 64, 16, 16, [(33, 33), (70, 500)], [20]),
    ("bf16", 128, 16, 1, [(130, 900)], []),
    ("fp8", 128, 32, 4, [(200, 1000)], [77]),
    # a short chunk deep into a long prompt: the context splits into ~128 ranges per tile
    ("bf16", 128, 16, 1, [(16, 40000)], [3]),
]


@pytest.mark.parametrize("kv,D,bs,G,chunks,dec", CHUNK_CASES,
                         ids=[f"{c[0]}-D{c[1]}-bs{c[2]}-G{c[3]}-{len(c[4])}ch" for c in CHUNK_CASES])
def test_prefill_chunk_small(kv, D, bs, G, chunks, dec):
    Hkv = 2
    _say(f"prefill case kv={kv} D={D} bs={bs} G={G} chunks={chunks} decodes={dec}")
    c = workloads.chunk_case("chunk", 200 + D + G, Hq=G * Hkv, Hkv=Hkv, D=D, bs=bs, chunks=chunks,
                             decode_lens=dec, kv_dtype=kv, std=1.0 if kv == "f32" else 0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    want = o.prefill()
    got = out_f64(g.chunk_out)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= tolerance(c), f"prefill max abs err {err:.3e}"
    if c.B:
        _check_decode(g, o)


# Context ranges longer than one 64-frame window of block ids: enough query tiles (a 512-row chunk
# over 8 KV heads) that the context splits only a few ways, so each range crosses two window
# switches and ends in a ragged window -- with 16-token bf16 frames (4 ranges of 2,304 keys, 144
# frames) and 32-token fp8 frames (2 ranges of 6,016 keys, 188 frames).
LONG_RANGE_CASES = [
    ("bf16", 16, 4, 9000),
    ("fp8", 32, 8, 12000),
]


@pytest.mark.parametrize("kv,bs,G,L", LONG_RANGE_CASES,
                         ids=[f"{c[0]}-bs{c[1]}-G{c[2]}-L{c[3]}" for c in LONG_RANGE_CASES])
def test_prefill_ranges_spanning_several_id_windows(kv, bs, G, L):
    Hkv = 8
    _say(f"long-range prefill kv={kv} bs={bs} G={G} chunk 512 at context {L}")
    c = workloads.chunk_case("long-range", 500 + bs + G, Hq=G * Hkv, Hkv=Hkv, D=128, bs=bs,
                             chunks=[(512, L)], decode_lens=[], kv_dtype=kv, std=0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    got = out_f64(g.chunk_out)
    assert np.isfinite(got).all()
    err = np.abs(got - o.prefill()).max()
    _say(f"  max abs err {err:.2e} over all 512 rows")
    assert err <= tolerance(c), f"prefill max abs err {err:.3e}"


def test_prefill_at_the_most_chunks_one_call_takes():
    """8,191 chunks of 1-16 rows over 8 kv heads (num_chunks x Hkv = 65,528, next to the call's
    limit of 65,535), each over a context of up to 60 earlier tokens: every output row."""
    _say("prefill with 8191 chunks")
    rng = np.random.default_rng(3)
    C = rng.integers(1, 17, size=8191)
    L = C + rng.integers(0, 61, size=8191)
    c = workloads.chunk_case("max-chunks", 13, Hq=16, Hkv=8, D=64, bs=16, chunks=list(zip(C, L)),
                             decode_lens=[], kv_dtype="bf16", std=0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    got = out_f64(g.chunk_out)
    assert np.isfinite(got).all()
    err = np.abs(got - o.prefill()).max()
    assert err <= tolerance(c), f"prefill max abs err {err:.3e}"


def test_copy_blocks_bit_exact_and_shared_equals_private():
    c = workloads.cases.fork_case("fork", 31, prompts=3, branches=4, prompt_len=64, tail_lo=3,
                                  tail_hi=70, Hq=16, Hkv=2, D=128, bs=32, kv_dtype="fp8")
    _say(f"copy_blocks case: {len(c.copy_pairs)} pairs")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    _check_decode(g, o)
    # a branch decoded through the shared prompt frames equals the same branch decoded through
    # private copies of them (bit for bit)
    first = g.out.clone()
    NB = c.NB
    extra = np.arange(NB, NB + 2 * c.block_tables.shape[1])
    kc2, vc2 = pa.new_kv_cache(NB + len(extra), c.Hkv, c.bs, c.D, c.kv_dtype, device=g.dev)
    kc2[:NB].copy_(g.kc)
    vc2[:NB].copy_(g.vc)
    row = c.block_tables[0].copy()
    n = -(-int(c.context_lens[0]) // c.bs)
    pairs = np.stack([row[:n], extra[:n]], 1).astype(np.int64)
    pa.copy_blocks(kc2, vc2, to_dev(pairs, "i64", g.dev), block_size=c.bs, kv_dtype=c.kv_dtype)
    tables = c.block_tables.copy()
    tables[0, :n] = extra[:n]
    out2 = pa.decode(g.q, kc2, vc2, to_dev(tables, "i32", g.dev), g.lens, block_size=c.bs,
                     scale=c.scale, kv_dtype=c.kv_dtype, max_context_len=c.max_context_len,
                     k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out2, first)


def test_frame_permutation_gives_identical_bits():
    c = workloads.decode_case("perm", 41, Hq=16, Hkv=2, D=128, bs=16, lens=[9, 300, 1400],
                              kv_dtype="bf16", std=0.7071, pool="scattered")
    g = GpuStep(c)
    g.step()
    base = g.out.clone()
    rng = np.random.default_rng(5)
    pi = rng.permutation(c.NB)
    inv = torch.from_numpy(np.argsort(pi)).to(g.dev)
    kc2 = g.kc[inv].contiguous()  # frame pi[f] of the new pool holds old frame f
    vc2 = g.vc[inv].contiguous()
    t2 = np.where(c.block_tables >= 0, pi[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    out2 = pa.decode(g.q, kc2, vc2, to_dev(t2, "i32", g.dev), g.lens, block_size=c.bs,
                     scale=c.scale, kv_dtype=c.kv_dtype, max_context_len=c.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(out2, base)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_nan_in_unwritten_tail_slots_never_leaks(kv):
    bs = 32 if kv == "fp8" else 16
    c = workloads.decode_case("nan", 43, Hq=8, Hkv=2, D=128, bs=bs, lens=[5, 37, 530],
                              kv_dtype=kv, std=0.7071, pool="scattered")
    g, o = GpuStep(c), OracleStep(c)
    # overwrite every slot past the context in each sequence's last frame with NaN
    nan_bits = np.full((1, c.Hkv, c.D), 0x7FC0, dtype=np.uint16)
    slots = []
    for b in range(c.B):
        L = int(c.context_lens[b])
        last = c.block_tables[b, (L - 1) // bs]
        slots += [int(last) * bs + t for t in range(L % bs or bs, bs)]
    if slots:
        nan_rows = to_dev(np.repeat(nan_bits, len(slots), 0), "bf16", g.dev)
        pa.reshape_and_cache(nan_rows, nan_rows, g.kc, g.vc,
                             torch.tensor(slots, dtype=torch.int64, device=g.dev), block_size=bs,
                             kv_dtype=kv, k_scale=c.k_scale, v_scale=c.v_scale)
    g.step()
    _check_decode(g, o)


def test_fp8_hardware_widening_matches_code_table():
    # V of a one-token context comes back exactly (p = 1): every finite e4m3fn code must
    # widen to its table value.
    table = oracle.e4m3fn_table()
    codes = np.array([cde if not np.isnan(table[cde]) else 0 for cde in range(256)])
    vals = table[codes].astype(np.float32).reshape(1, 2, 128)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits).ravel(), table[codes])
    dev = device()
    kc, vc = pa.new_kv_cache(4, 2, 32, 128, "fp8", device=dev)
    kc.zero_()
    vc.zero_()
    rows = to_dev(bits, "bf16", dev)
    pa.reshape_and_cache(rows, rows, kc, vc, torch.tensor([64], dtype=torch.int64, device=dev),
                         block_size=32, kv_dtype="fp8", k_scale=1.0, v_scale=1.0)
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device=dev)
    out = pa.decode(q, kc, vc, torch.tensor([[2]], dtype=torch.int32, device=dev),
                    torch.tensor([1], dtype=torch.int32, device=dev), block_size=32, scale=0.1,
                    kv_dtype="fp8", max_context_len=1)
    torch.cuda.synchronize()
    stored = to_raw(vc)[2, :, :].reshape(2, -1)
    vpos = oracle.tile_positions("v", 32, 128, "fp8")
    np.testing.assert_array_equal(stored[:, vpos[0]], codes.reshape(2, 128))
    np.testing.assert_array_equal(out_f64(out).ravel(), table[codes])


def test_fp8_encode_matches_oracle_bits():
    rng = np.random.default_rng(44)
    t = oracle.e4m3fn_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 448.0, 449.0, 464.0, 500.0, 1e9, np.inf, -np.inf, np.nan,
                        2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -12], dtype=np.float32)
    x = np.concatenate([mids, -mids, special, (rng.standard_normal(256 * 8 - 2 * len(mids) -
                                                                  len(special)) * 50).astype(np.float32)])
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rows = bits.reshape(16, 1, 128)
    dev = device()
    kc, vc = pa.new_kv_cache(2, 1, 16, 128, "fp8", device=dev)
    slots = np.arange(16, dtype=np.int64)
    for scale in (1.0, 0.37):
        pa.reshape_and_cache(to_dev(rows, "bf16", dev), to_dev(rows, "bf16", dev), kc, vc,
                             to_dev(slots, "i64", dev), block_size=16, kv_dtype="fp8",
                             k_scale=scale, v_scale=2.5)
        torch.cuda.synchronize()
        okc = oracle.new_cache(2, 1, 16, 128, "fp8")
        ovc = oracle.new_cache(2, 1, 16, 128, "fp8")
        oracle.reshape_and_cache(okc, ovc, rows, rows, slots, bs=16, src_dtype="bf16",
                                 kv_dtype="fp8", k_scale=scale, v_scale=2.5)
        np.testing.assert_array_equal(to_raw(kc)[0], okc[0])
        np.testing.assert_array_equal(to_raw(vc)[0], ovc[0])


def test_negative_slots_are_skipped_and_other_frames_untouched():
    dev = device()
    kc, vc = pa.new_kv_cache(3, 2, 16, 64, "f32", device=dev)
    kc.fill_(7.0)
    vc.fill_(-7.0)
    rows = torch.randn(4, 2, 64, device=dev)
    pa.reshape_and_cache(rows, rows, kc, vc, torch.tensor([-1, 17, -5, 18], device=dev),
                         block_size=16, kv_dtype="f32")
    torch.cuda.synchronize()
    okc = np.full((3, 2, 16 * 64), 7.0, np.float32)
    ovc = np.full((3, 2, 16 * 64), -7.0, np.float32)
    oracle.reshape_and_cache(okc, ovc, rows.cpu().numpy(), rows.cpu().numpy(),
                             np.array([-1, 17, -5, 18]), bs=16, src_dtype="f32", kv_dtype="f32")
    np.testing.assert_array_equal(to_raw(kc), okc)
    np.testing.assert_array_equal(to_raw(vc), ovc)


def test_one_token_and_identical_keys_closed_forms_on_gpu():
    dev = device()
    D, bs, Hkv, G = 128, 16, 2, 4
    L = 777
    nblk = -(-L // bs)
    kc, vc = pa.new_kv_cache(nblk + 1, Hkv, bs, D, "bf16", device=dev)
    rng = np.random.default_rng(3)
    krow = torch.from_numpy(rng.standard_normal((1, Hkv, D)).astype(np.float32)).bfloat16()
    vrows = torch.from_numpy(rng.standard_normal((L, Hkv, D)).astype(np.float32)).bfloat16()
    slots = torch.arange(L, dtype=torch.int64) + bs  # frames 1..nblk
    pa.reshape_and_cache(krow.repeat(L, 1, 1).to(dev), vrows.to(dev), kc, vc, slots.to(dev),
                         block_size=bs, kv_dtype="bf16")
    q = torch.from_numpy(rng.standard_normal((2, Hkv * G, D)).astype(np.float32)).bfloat16().to(dev)
    tables = torch.tensor([list(range(1, nblk + 1)), [1] + [0] * (nblk - 1)], dtype=torch.int32, device=dev)
    out = pa.decode(q, kc, vc, tables, torch.tensor([L, 1], dtype=torch.int32, device=dev),
                    block_size=bs, scale=1 / math.sqrt(D), kv_dtype="bf16", max_context_len=L)
    torch.cuda.synchronize()
    o = out_f64(out)
    mean = vrows.double().mean(0).numpy()
    for h in range(Hkv * G):
        assert np.abs(o[0, h] - mean[h // G]).max() < 4e-3
        np.testing.assert_array_equal(o[1, h], vrows[0, h // G].double().numpy())


# The decode launch is sized from the host-known bound B Hkv (ceil(max_context_len / bs) + 4) at
# 16 units per wavefront (whole workgroups of 4, at most 3 per compute unit): these batches give
# launches from the smallest through intermediate sizes, with lengths that cut runs at many
# wavefront boundaries.  (The first takes the run-aligned launch below: one wavefront per run.)
LAUNCH_SIZE_CASES = [
    # (B, longest length drawn, G)
    (1, 40, 8),
    (3, 700, 8),
    (9, 1500, 8),
    (24, 3000, 8),
    (40, 4096, 8),
]


@pytest.mark.parametrize("B,maxlen,G", LAUNCH_SIZE_CASES,
                         ids=[f"B{c[0]}-L{c[1]}" for c in LAUNCH_SIZE_CASES])
def test_decode_launch_sizes(B, maxlen, G):
    Hkv = 2
    _say(f"decode launch-size case B={B} max length {maxlen}")
    c = workloads.decode_case("launch-size", 900 + B, Hq=G * Hkv, Hkv=Hkv, D=128, bs=16,
                              lens=lambda rng: rng.integers(1, maxlen + 1, size=B),
                              kv_dtype="bf16", std=0.7071)
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    _check_decode(g, o)


def _stream_wavefronts() -> int:
    """Wavefronts of a full decode stream launch on this device: 3 per compute unit, in whole
    workgroups of 4."""
    return torch.cuda.get_device_properties(0).multi_processor_count * 3 // 4 * 4


# A batch whose runs have at most 28 frames by the host-known bound (ceil(max_context_len / bs)
# + 4 <= 32 units) and whose B Hkv runs fit in the stream's wavefronts launches one wavefront per
# (sequence, kv head) run, each writing its output directly, and no merge.  One frame more, or
# one run more than the stream holds, takes the split launch.  Cases on both sides of each bound;
# every output against the oracle.
ALIGNED_CASES = [
    # (name, B, Hq, Hkv, D, bs, kv, longest length; B = 0: the stream's wavefronts / Hkv (+1))
    ("aligned-f32-D64", 5, 8, 4, 64, 16, "f32", 448),
    ("aligned-bf16", 6, 16, 2, 128, 16, "bf16", 448),
    ("aligned-fp8-bs32", 7, 64, 8, 128, 32, "fp8", 896),
    ("split-one-frame-past-f32-D64", 5, 8, 4, 64, 16, "f32", 449),
    ("split-one-frame-past-fp8-bs32", 7, 64, 8, 128, 32, "fp8", 897),
    ("aligned-runs-fill-the-stream", 0, 16, 2, 128, 16, "bf16", 448),
    ("split-one-sequence-past-the-stream", -1, 16, 2, 128, 16, "bf16", 448),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,bs,kv,longest", ALIGNED_CASES,
                         ids=[c[0] for c in ALIGNED_CASES])
def test_decode_run_aligned_bounds(name, B, Hq, Hkv, D, bs, kv, longest):
    if B <= 0:
        B = _stream_wavefronts() // Hkv + (1 if B < 0 else 0)
    _say(f"run-aligned bound case {name}: B={B} Hkv={Hkv} longest {longest}")

    def lens(rng):
        x = rng.integers(1, longest + 1, size=B)
        x[rng.integers(B)] = longest
        return x

    c = workloads.decode_case(name, 40 + B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens, kv_dtype=kv,
                              std=1.0 if kv == "f32" else 0.7071, pool="scattered")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    _check_decode(g, o)


STREAM_CASES = [
    # (name, Hq, Hkv, kv, bs, lengths): extremes of the batch-wide stream split
    ("one-sequence-over-every-wavefront", 8, 1, "bf16", 16, [100000]),
    ("thousands-of-tiny-sequences", 8, 2, "bf16", 16, "tiny"),
    ("long-and-tiny-mix-fp8", 16, 2, "fp8", 32, [1, 2, 40000, 3, 17, 33]),
    # the largest batch planned inside the stream kernel's wavefronts, and the smallest one
    # planned by the separate plan kernel
    ("batch-1024-wave-planned", 8, 2, "bf16", 16, "b1024"),
    ("batch-1025-kernel-planned", 8, 2, "bf16", 16, "b1025"),
]


@pytest.mark.parametrize("name,Hq,Hkv,kv,bs,lens", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_decode_stream_split_extremes(name, Hq, Hkv, kv, bs, lens):
    _say(f"stream case {name}")
    if lens == "tiny":
        lens = lambda rng: rng.integers(1, 41, size=3000)
    elif lens in ("b1024", "b1025"):
        nb = int(lens[1:])
        lens = lambda rng: rng.integers(1, 400, size=nb)
    c = workloads.decode_case(name, 7, Hq=Hq, Hkv=Hkv, D=128, bs=bs, lens=lens, kv_dtype=kv,
                              std=0.7071, pool="scattered")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_decode(g, o)


def test_decode_at_the_largest_batch_one_call_takes():
    """65,535 sequences (the most one pa_decode call accepts) of 1-40 tokens, planned by the
    separate plan kernel: every cache slot bit-exact and every output against the oracle."""
    _say("max batch 65535")
    c = workloads.decode_case("max-batch", 11, Hq=4, Hkv=1, D=64, bs=16,
                              lens=lambda rng: rng.integers(1, 41, size=65535), kv_dtype="bf16",
                              std=0.7071, pool="scattered")
    g, o = GpuStep(c), OracleStep(c)
    g.step()
    _check_caches(g, o)
    _check_decode(g, o)


def test_graph_replays_match_eager_bits():
    """A step captured in a HIP graph (copies, cache writes, prefill chunk, decode, and the mixed
    step in its single-kernel mode) and replayed several times, with eager work between the
    replays, gives the eager step's bits each time."""
    _say("graph replay case")
    c = workloads.fork_case("graph-fork", 11, prompts=3, branches=3, prompt_len=320, tail_lo=1,
                            tail_hi=60, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16")
    g = GpuStep(c)
    ch = workloads.chunk_case("graph-chunk", 12, Hq=16, Hkv=2, D=128, bs=16,
                              chunks=[(33, 200), (70, 900)], decode_lens=[5, 400, 1200],
                              kv_dtype="bf16", std=0.7071)
    h = GpuStep(ch)
    dev = g.dev
    ws = torch.empty(pa.decode_workspace_bytes(c.B, c.Hq, c.D, c.bs, c.kv_dtype,
                                               c.max_context_len), dtype=torch.uint8, device=dev)
    out = torch.empty_like(g.q)
    cout = torch.empty_like(h.cq)
    mout = torch.empty((h.c.B + h.cq.shape[0],) + tuple(h.cq.shape[1:]), dtype=h.cq.dtype,
                       device=dev)

    def step():
        g.write()
        g.decode(out=out, workspace=ws)
        h.write()
        h.prefill()
        cout.copy_(h.chunk_out)
        h.mixed(mode="split")
        mout.copy_(h.mixed_out)

    step()
    torch.cuda.synchronize()
    want, cwant, mwant = out.clone(), cout.clone(), mout.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        cout.zero_()
        mout.zero_()
        # eager work between the replays: another decode into a fresh buffer
        g.decode()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"decode, replay {r}"
        assert torch.equal(cout.view(torch.int16), cwant.view(torch.int16)), f"prefill, replay {r}"
        assert torch.equal(mout.view(torch.int16), mwant.view(torch.int16)), f"mixed, replay {r}"
    o = OracleStep(c)
    err = np.abs(out_f64(out) - o.decode()).max()
    assert err <= tolerance(c)


@pytest.mark.parametrize("shared", ["fork", "plain"])
def test_shared_frames_hint_gives_identical_bits(shared):
    """The cache-policy flag changes only where tiles are cached: both settings, bit for bit."""
    _say(f"shared-frames hint, {shared} case")
    if shared == "fork":
        c = workloads.fork_case("hint-fork", 5, prompts=4, branches=4, prompt_len=256, tail_lo=1,
                                tail_hi=100, Hq=32, Hkv=4, D=128, bs=32, kv_dtype="fp8")
    else:
        c = workloads.decode_case("hint-plain", 5, Hq=16, Hkv=2, D=128, bs=16,
                                  lens=[1, 100, 1000, 3000], kv_dtype="bf16", std=0.7071)
    g = GpuStep(c)
    g.write()
    a = g.decode(shared_frames=False).clone()
    b = g.decode(shared_frames=True).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert c.shares_frames == (shared == "fork")
    o = OracleStep(c)
    assert np.abs(out_f64(b) - o.decode()).max() <= tolerance(c)


def test_prepared_calls_match_ordinary_calls_bit_for_bit():
    c = workloads.chunk_case("prepared", 77, Hq=16, Hkv=4, D=128, bs=16, chunks=[(96, 700)],
                             decode_lens=[5, 300, 1200, 2048], kv_dtype="fp8", std=0.7071)
    g = GpuStep(c)
    g.write()
    d0 = g.decode().clone()
    c0 = g.prefill().clone()
    _, m0 = g.mixed(mode="split")
    m0 = m0.clone()
    ws = torch.empty(pa.decode_workspace_bytes(c.B, c.Hq, c.D, c.bs, c.kv_dtype,
                                               c.max_context_len), dtype=torch.uint8,
                     device=g.dev)
    out = torch.zeros_like(g.q)
    call = pa.decode(g.q, g.kc, g.vc, g.tables, g.lens, block_size=c.bs, scale=c.scale,
                     kv_dtype=c.kv_dtype, max_context_len=c.max_context_len, k_scale=c.k_scale,
                     v_scale=c.v_scale, out=out, workspace=ws, prepared=True)
    assert isinstance(call, pa.PreparedCall) and not out.any()
    ch = c.chunk
    cws = torch.empty(max(1, pa.prefill_chunk_workspace_bytes(
        ch.num_chunks, g.cq.shape[0], ch.max_chunk_len, ch.max_context_len, c.Hq, c.Hkv, c.D,
        c.bs, c.kv_dtype)), dtype=torch.uint8, device=g.dev)
    cout = torch.zeros_like(g.cq)
    pcall = pa.prefill_chunk(g.cq, g.kc, g.vc, g.ctables, g.cqsl, g.clens, block_size=c.bs,
                             scale=c.scale, kv_dtype=c.kv_dtype, max_chunk_len=ch.max_chunk_len,
                             max_context_len=ch.max_context_len, k_scale=c.k_scale,
                             v_scale=c.v_scale, out=cout, workspace=cws, prepared=True)
    for _ in range(2):
        call()
        pcall()
        torch.cuda.synchronize()
        assert torch.equal(out, d0)
        assert torch.equal(cout, c0)
    _, m1 = g.mixed(mode="split")
    torch.cuda.synchronize()
    assert torch.equal(m1, m0)


def test_empty_calls_are_no_ops():
    """Every entry point accepts an empty batch (no tokens, sequences, chunks or copy pairs):
    the call succeeds, writes nothing, and the next non-empty call on the stream is unaffected."""
    _say("empty calls")
    dev = device()
    NB, Hkv, Hq, D, bs = 8, 2, 4, 128, 16
    kc, vc = pa.new_kv_cache(NB, Hkv, bs, D, "bf16", device=dev)
    kc.fill_(1.5)
    vc.fill_(-2.5)
    before_k, before_v = to_raw(kc).copy(), to_raw(vc).copy()
    none_rows = torch.empty(0, Hkv, D, dtype=torch.bfloat16, device=dev)
    pa.reshape_and_cache(none_rows, none_rows, kc, vc,
                         torch.empty(0, dtype=torch.int64, device=dev), block_size=bs,
                         kv_dtype="bf16")
    pa.copy_blocks(kc, vc, torch.empty(0, 2, dtype=torch.int64, device=dev), block_size=bs,
                   kv_dtype="bf16")
    q0 = torch.empty(0, Hq, D, dtype=torch.bfloat16, device=dev)
    bt0 = torch.empty(0, 4, dtype=torch.int32, device=dev)
    lens0 = torch.empty(0, dtype=torch.int32, device=dev)
    assert pa.decode_workspace_bytes(0, Hq, D, bs, "bf16", 64) == 0
    out = pa.decode(q0, kc, vc, bt0, lens0, block_size=bs, scale=0.1, kv_dtype="bf16",
                    max_context_len=64)
    assert out.shape == (0, Hq, D)
    qsl0 = torch.zeros(1, dtype=torch.int32, device=dev)
    pa.prefill_chunk(q0, kc, vc, bt0, qsl0, lens0, block_size=bs, scale=0.1, kv_dtype="bf16",
                     max_chunk_len=16, max_context_len=64)
    for mode in ("auto", "split", "separate"):
        pa.mixed_attention(q0, kc, vc, bt0, qsl0, lens0, 0, block_size=bs, scale=0.1,
                           kv_dtype="bf16", max_chunk_len=16, max_context_len=64, mode=mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_raw(kc), before_k)
    np.testing.assert_array_equal(to_raw(vc), before_v)
    # a one-token decode right after: the output is that token's V row (closed form)
    q1 = torch.randn(1, Hq, D, device=dev).to(torch.bfloat16)
    bt1 = torch.tensor([[3, 0, 0, 0]], dtype=torch.int32, device=dev)
    out1 = pa.decode(q1, kc, vc, bt1, torch.tensor([1], dtype=torch.int32, device=dev),
                     block_size=bs, scale=0.1, kv_dtype="bf16", max_context_len=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_f64(out1), np.full((1, Hq, D), -2.5))
