"""Invariants of the seeded synthetic inputs (host only, small and medium cases)."""

import numpy as np
import pytest

import workloads
from workloads import cases


def _check_tables(c, shared_ok=False):
    used = []
    for b in range(c.B):
        L = int(c.context_lens[b])
        nblk = -(-L // c.bs)
        row = c.block_tables[b]
        assert np.all(row[:nblk] >= 0) and np.all(row[:nblk] < c.NB)
        assert np.all(row[nblk:] == -1)
        # waste is confined to the last block: fewer than bs unused slots per sequence
        assert 0 <= nblk * c.bs - L < c.bs
        used.extend(row[:nblk].tolist())
    if not shared_ok:
        assert len(used) == len(set(used))


def test_config1_fixed_shape():
    c = workloads.make(1)
    assert (c.B, c.Hq, c.Hkv, c.D, c.bs, c.NB) == (4, 4, 2, 64, 16, 64)
    assert c.context_lens.tolist() == [1, 17, 100, 255]
    assert c.q_dtype == c.kv_dtype == "f32" and c.scale == 1 / 8
    _check_tables(c)
    # the new token sits at position L-1: (logical block, offset) (0,0), (1,0), (6,3), (15,14)
    for b, (lb, off) in enumerate([(0, 0), (1, 0), (6, 3), (15, 14)]):
        assert c.new_slots[b] == c.block_tables[b, lb] * 16 + off
    # 26 frames used, the other 38 hold poison only
    assert int((-(-c.context_lens // 16)).sum()) == 26
    live = c.meta["live_slots"]
    assert live == int(c.context_lens.sum()) - c.B


def test_reproducible_draws():
    a = workloads.decode_case("x", 7, Hq=8, Hkv=2, D=64, bs=16, lens=[5, 40], kv_dtype="bf16")
    b = workloads.decode_case("x", 7, Hq=8, Hkv=2, D=64, bs=16, lens=[5, 40], kv_dtype="bf16")
    for f in ("q", "pool_k", "pool_v", "new_k", "new_v", "block_tables", "new_slots"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_poison_marks_every_non_live_slot():
    c = workloads.decode_case("x", 3, Hq=8, Hkv=2, D=64, bs=16, lens=[1, 16, 17, 40],
                              kv_dtype="f32", pool=12)
    live = np.zeros(c.NB * c.bs, bool)
    for b in range(c.B):
        L = int(c.context_lens[b])
        t = np.arange(L - 1)
        live[c.block_tables[b, t // 16].astype(np.int64) * 16 + t % 16] = True
    assert np.all(c.pool_k[~live] == workloads.POISON_K)
    assert np.all(c.pool_v[~live] == workloads.POISON_V)
    assert not np.any(c.pool_v[live] == workloads.POISON_V)
    assert np.all(c.pool_k[c.new_slots] == workloads.POISON_K)


def test_fork_case_sharing_and_copy_pairs():
    c = cases.fork_case("f", 4, prompts=3, branches=4, prompt_len=64, tail_lo=3, tail_hi=70,
                        Hq=8, Hkv=2, D=64, bs=32)
    _check_tables(c, shared_ok=True)
    pf = c.meta["prompt_frames"]
    for b in range(c.B):
        np.testing.assert_array_equal(c.block_tables[b, :2], pf[b // 4])
    src, dst = c.copy_pairs[:, 0], c.copy_pairs[:, 1]
    assert len(set(dst.tolist())) == len(dst) and not set(src.tolist()) & set(dst.tolist())
    # every copy source is a shared, partially filled tail frame; every destination is fresh
    # and the branch's table points at the destination where its new token goes
    for b in range(c.B):
        pos = int(c.context_lens[b]) - 1
        frame = c.block_tables[b, pos // 32]
        assert c.new_slots[b] == frame * 32 + pos % 32
        if pos % 32:
            assert frame in dst
    assert np.all(c.pool_k[dst.astype(np.int64)[:, None] * 32 + np.arange(32)] ==
                  cases._const(workloads.POISON_K, "bf16"))
    assert 0 < c.k_scale < 1 and 0 < c.v_scale < 1


def test_chunk_case_positions():
    c = workloads.chunk_case("c", 5, Hq=8, Hkv=2, D=64, bs=16, chunks=[(20, 70), (16, 16)],
                             decode_lens=[5, 33])
    ch = c.chunk
    assert ch.query_start_loc.tolist() == [0, 20, 36]
    assert ch.context_lens.tolist() == [70, 16]
    # the chunks' tokens are the first rows of the step's writes, at positions L-C .. L-1
    t = np.arange(50, 70)
    np.testing.assert_array_equal(c.new_slots[:20], ch.block_tables[0, t // 16] * 16 + t % 16)
    assert c.new_slots.shape[0] == 20 + 16 + 2


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 4])
def test_named_configs_shapes(cfg):
    c = workloads.make(cfg)
    _check_tables(c, shared_ok=(cfg == 4))
    if cfg == 2:
        assert (c.B, c.Hq, c.Hkv, c.D, c.bs) == (64, 32, 8, 128, 16)
        assert c.context_lens.min() >= 512 and c.context_lens.max() <= 4096
        assert c.NB == int((-(-c.context_lens // 16)).sum())
    else:
        assert (c.B, c.Hq, c.Hkv, c.D, c.bs, c.kv_dtype) == (256, 64, 8, 128, 32, "fp8")
        assert np.all((c.context_lens >= 1024 + 64) & (c.context_lens <= 1024 + 512))
        assert 200 < len(c.copy_pairs) <= 256


def _scaled_scores(c, b, head):
    """Host-side scaled scores (log2 of the softmax weights, before the shift) of sequence b's
    keys for query head `head`, from the case's raw inputs (the keys of positions < L-1 are in
    the pool, the last one is the step's new row)."""
    L = int(c.context_lens[b])
    t = np.arange(L - 1)
    slots = c.block_tables[b, t // c.bs].astype(np.int64) * c.bs + t % c.bs
    g = head // c.G
    k = np.concatenate([cases._as_f32(c.pool_k[slots, g], c.src_dtype),
                        cases._as_f32(c.new_k[b:b + 1, g], c.src_dtype)]).astype(np.float64)
    q = cases._as_f32(c.q[b, head], c.q_dtype).astype(np.float64)
    return c.scale * np.log2(np.e) * (k @ q)


@pytest.mark.parametrize("profile", workloads.SCORE_PROFILES)
def test_steered_scores_follow_their_profile(profile):
    base = workloads.decode_case("steer", 12, Hq=8, Hkv=2, D=128, bs=16, lens=[40, 700, 2100],
                                 kv_dtype="bf16", std=0.7071, pool="scattered")
    c = workloads.steer_scores(base, 5, profile)
    t_max = 2099
    for head in (0, 5):
        s = _scaled_scores(c, 2, head)
        if profile == "rising":
            assert s[-1] - s[0] > 0.9 * 60.0 and np.corrcoef(np.arange(len(s)), s)[0, 1] > 0.99
        elif profile == "falling":
            assert s[0] - s[-1] > 0.9 * 60.0 and np.corrcoef(np.arange(len(s)), s)[0, 1] < -0.99
        else:
            top = (3 * t_max) // 4
            others = np.delete(s, top)
            assert s[top] - others.max() > 24.0  # the span/2 spike at t_max // 3 is the next
            assert s[top] - np.median(others) > 55.0
    # only the queries and keys change: values, tables and the poison stay
    np.testing.assert_array_equal(c.pool_v, base.pool_v)
    np.testing.assert_array_equal(c.block_tables, base.block_tables)
    dead = np.ones(c.NB * c.bs, bool)
    for b in range(c.B):
        t = np.arange(int(c.context_lens[b]) - 1)
        dead[c.block_tables[b, t // c.bs].astype(np.int64) * c.bs + t % c.bs] = False
    np.testing.assert_array_equal(c.pool_k[dead], base.pool_k[dead])


def test_steered_scores_fp8_scales_cover_the_new_keys():
    base = workloads.decode_case("steer8", 13, Hq=8, Hkv=2, D=128, bs=32, lens=[100, 1500],
                                 kv_dtype="fp8", std=0.7071, pool="scattered")
    c = workloads.steer_scores(base, 6, "rising")
    live = np.zeros(c.NB * c.bs, bool)
    for b in range(c.B):
        t = np.arange(int(c.context_lens[b]) - 1)
        live[c.block_tables[b, t // c.bs].astype(np.int64) * c.bs + t % c.bs] = True
    amax = max(np.abs(cases._as_f32(c.pool_k[live], "bf16")).max(),
               np.abs(cases._as_f32(c.new_k, "bf16")).max())
    assert c.k_scale == pytest.approx(amax / 448.0, rel=1e-6)
    assert c.v_scale == base.v_scale
