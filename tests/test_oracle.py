"""Pins of the CPU reference (oracle/) against what the pages and the mathematics fix.

No GPU and no part of the HIP library is involved.  Each test names the
passage or the closed form it checks; test_mutations.py shows that plausible
mistakes in the reference fail at least one of these checks.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.layout import tile_positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- helpers


def _store(tokens_k, tokens_v, tables, lens, *, bs, NB, kv_dtype="f32", src_dtype="f32",
           k_scale=1.0, v_scale=1.0):
    """Caches holding each sequence's tokens (rows of tokens_k[b][t]) through its table."""
    Hkv, D = tokens_k[0].shape[1:]
    kc = oracle.new_cache(NB, Hkv, bs, D, kv_dtype)
    vc = oracle.new_cache(NB, Hkv, bs, D, kv_dtype)
    for b, L in enumerate(lens):
        slots = oracle.slot_of(tables[b], np.arange(L), bs)
        oracle.reshape_and_cache(kc, vc, tokens_k[b][:L], tokens_v[b][:L], slots, bs=bs,
                                 src_dtype=src_dtype, kv_dtype=kv_dtype, k_scale=k_scale,
                                 v_scale=v_scale)
    return kc, vc


def _sdpa(q, K, V, scale, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU, KV heads repeated G times.
    q [Hq, Lq, D], K/V [L, Hkv, D]."""
    Hq, Hkv = q.shape[0], K.shape[1]
    G = Hq // Hkv
    k = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, 0)
    v = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, 0)
    qq = torch.from_numpy(np.ascontiguousarray(q))
    return torch.nn.functional.scaled_dot_product_attention(
        qq[None], k[None], v[None], scale=scale, is_causal=causal)[0].numpy()


def _rand_tokens(rng, B, L, Hkv, D, std=1.0):
    return ([rng.standard_normal((L, Hkv, D)).astype(np.float32) * np.float32(std) for _ in range(B)],
            [rng.standard_normal((L, Hkv, D)).astype(np.float32) * np.float32(std) for _ in range(B)])


def _identity_tables(B, maxblk):
    return np.arange(B * maxblk, dtype=np.int32).reshape(B, maxblk)


# ----------------------------------------------------------------------------- KV-size arithmetic


def test_kv_size_equation_as_printed():
    g = _golden("page_examples.json")["kv_size_equation"]
    n = oracle.kv_bytes_per_token_page_formula(g["n_layers"], g["n_kv_heads"], g["d_head"], g["bytes"])
    assert n == g["bytes_per_token"] == 655360
    assert n * g["tokens"] > g["sequence_bytes_exceeds"]


def test_vram_math_per_layer():
    g = _golden("page_examples.json")["vram_math_llama2_7b"]
    per_layer = oracle.kv_bytes_per_token_per_layer_p3(g["head_size"], g["num_heads"], g["dtype_bytes"])
    assert per_layer == g["bytes_per_token_per_layer"]
    assert per_layer * g["num_layers"] == g["bytes_per_token"]


def test_physical_cache_bytes_per_token():
    # One 70B layer: 8 KV heads of 128 in bf16 occupy 4096 bytes per token in k_cache + v_cache;
    # over 80 layers that is half of the printed equation (its extra factor of 2).
    NB, bs = 3, 16
    kc = oracle.new_cache(NB, 8, bs, 128, "bf16")
    vc = oracle.new_cache(NB, 8, bs, 128, "bf16")
    per_tok = (kc.nbytes + vc.nbytes) // (NB * bs)
    assert per_tok == oracle.kv_bytes_per_token_layer(8, 128, "bf16") == 4096
    assert per_tok * 80 * 2 == oracle.kv_bytes_per_token_page_formula(80, 8, 128, 2)
    assert oracle.kv_bytes_per_token_layer(8, 128, "fp8") == 2048


# ----------------------------------------------------------------------------- number formats


def test_bf16_decode_closed_form_and_torch():
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049])).tolist()[:4] == \
        [1.0, -2.0, 0.0, -0.0]
    assert oracle.bf16_bits_to_f64(np.array([0x4049]))[0] == 3.140625
    bits = np.random.default_rng(0).integers(0, 1 << 16, 5000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_e4m3fn_table_closed_form():
    t = oracle.e4m3fn_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) == -1
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3fn_table_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.e4m3fn_table()
    fin = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert np.all(np.isnan(ref[~fin]))


def test_e4m3fn_encode_in_range_matches_torch_rne():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(20000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3fn_encode(y), ref)


def test_e4m3fn_encode_ties_saturation_nan():
    t = oracle.e4m3fn_table()
    # exact midpoints between neighbouring codes go to the even code
    for c in range(0, 0x7E):
        mid = np.float32((t[c] + t[c + 1]) / 2)
        assert float(mid) == (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3fn_encode(np.array([mid]))[0] == want
        assert oracle.e4m3fn_encode(np.array([-mid]))[0] == want | 0x80
    big = np.array([448.0, 449.0, 464.0, 500.0, 1e6, np.inf, -np.inf, -1e30], dtype=np.float32)
    assert oracle.e4m3fn_encode(big).tolist() == [0x7E] * 6 + [0xFE, 0xFE]
    assert oracle.e4m3fn_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    assert oracle.e4m3fn_encode(np.array([-0.0], np.float32))[0] == 0x80


def test_fp8_store_error_bound():
    # Round to nearest with a 3-bit mantissa: |decode(encode(y)) - y| <= 2^-4 |y| for normal
    # magnitudes, <= 2^-10 absolute in the subnormal range, and the result is a nearest code.
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(50000) * 40).astype(np.float32)
    y = y[np.abs(y) <= 448]
    back = oracle.e4m3fn_decode(oracle.e4m3fn_encode(y))
    err = np.abs(back - y.astype(np.float64))
    bound = np.maximum(np.abs(y.astype(np.float64)) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound)
    t = oracle.e4m3fn_table()[:0x7F]
    nearest = np.min(np.abs(np.abs(y.astype(np.float64))[:, None] - t[None, :]), axis=1)
    np.testing.assert_array_equal(err, nearest)


# ----------------------------------------------------------------------------- tile layout


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("dtype,bs,D", [("f32", 16, 64), ("f32", 16, 128), ("bf16", 16, 64),
                                        ("bf16", 16, 128), ("bf16", 32, 128), ("fp8", 16, 128),
                                        ("fp8", 32, 128), ("fp8", 32, 64)])
def test_tile_layout_is_bijection(kind, dtype, bs, D):
    pos = tile_positions(kind, bs, D, dtype)
    assert sorted(pos.ravel().tolist()) == list(range(bs * D))


def test_tile_layout_hand_evaluated_entries():
    for c in _golden("tile_layout.json")["cases"]:
        pos = tile_positions(c["kind"], c["bs"], c["D"], c["dtype"])
        assert pos[c["o"], c["d"]] == c["elem"], c


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(3)
    vals = rng.integers(0, 1 << 16, (5, 3, 16, 128)).astype(np.uint16)
    for kind in "kv":
        tiles = oracle.pack_tiles(vals, kind, "bf16")
        np.testing.assert_array_equal(oracle.unpack_tiles(tiles, kind, "bf16", 16, 128), vals)


# ----------------------------------------------------------------------------- block tables and slots


def test_slot_of_follows_the_block_split_rule():
    """codebumble.net, "The Block Table Mapping Subsystem": a position's logical block is
    position // block_size and its offset position % block_size, and a sequence takes the next
    frame from the head of a FIFO free list whenever it opens a block.  The frames that rule
    hands out are written here in closed form instead of being simulated."""
    g = _golden("page_examples.json")["allocate_slot"]
    bs = g["block_size"]
    # one sequence of 48 tokens from a fresh pool opens blocks 0, 1, 2 and takes frames 0, 1, 2
    table = np.array(g["first_sequence_frames"], dtype=np.int32)
    for pos in range(48):
        assert oracle.slot_of(table, [pos], bs)[0] == [0, 1, 2][pos // 16] * 16 + pos % 16
    # two sequences r = 0, 1 growing in lockstep open their j-th blocks one after the other, so
    # sequence r's block j holds frame 2 j + r
    for r in (0, 1):
        tab = np.array([2 * j + r for j in range(3)], dtype=np.int32)
        pos = np.arange(40)
        want = (2 * (pos // 16) + r) * 16 + pos % 16
        np.testing.assert_array_equal(oracle.slot_of(tab, pos, bs), want)
    # a vector of positions is split element by element, and int64 holds slots past 2^31
    big = np.array([2 ** 27, 5], dtype=np.int32)
    assert oracle.slot_of(big, [3], bs)[0] == 2 ** 31 + 3
    assert oracle.slot_of(big, [17], bs)[0] == 5 * 16 + 1


@pytest.mark.parametrize("which", ["block_table_codebumble", "block_table_bicarait"])
def test_diagram_block_tables(which):
    g = _golden("page_examples.json")[which]
    bs, n, frames = g["block_size"], g["tokens"], g["frames"]
    table = np.array(frames, dtype=np.int32)
    # tokens 0-15, 16-31, 32-47 land in the three listed frames
    for t in (0, 15, 16, 31, 32, 47):
        assert oracle.slot_of(table, [t], bs)[0] == frames[t // bs] * bs + t % bs
    # attention through that table equals attention over the contiguous tokens
    rng = np.random.default_rng(4)
    Hkv, Hq, D = 2, 4, 64
    tk, tv = _rand_tokens(rng, 1, n, Hkv, D)
    kc, vc = _store(tk, tv, table[None], [n], bs=bs, NB=max(frames) + 1)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, table[None], np.array([n]), scale=0.125, bs=bs,
                        q_dtype="f32", kv_dtype="f32")
    ref = _sdpa(q[0][:, None, :].astype(np.float64), tk[0].astype(np.float64),
                tv[0].astype(np.float64), 0.125)[:, 0]
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- decode


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 1), (8, 8), (32, 8)])
def test_identity_table_equals_textbook_attention(Hq, Hkv):
    rng = np.random.default_rng(5)
    D, bs, lens = 64, 16, [1, 17, 100, 48]
    maxblk = 7
    tk, tv = _rand_tokens(rng, len(lens), maxblk * bs, Hkv, D)
    tables = _identity_tables(len(lens), maxblk)
    kc, vc = _store(tk, tv, tables, lens, bs=bs, NB=len(lens) * maxblk)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, tables, np.array(lens), scale=0.125, bs=bs, q_dtype="f32",
                        kv_dtype="f32")
    for b, L in enumerate(lens):
        ref = _sdpa(q[b][:, None, :].astype(np.float64), tk[b][:L].astype(np.float64),
                    tv[b][:L].astype(np.float64), 0.125)[:, 0]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_frame_permutation_invariance():
    rng = np.random.default_rng(6)
    D, bs, lens, NB = 128, 16, [33, 70, 5], 16
    Hkv, Hq = 2, 8
    perm0 = rng.permutation(NB)
    nblk = [-(-L // bs) for L in lens]
    tables = np.full((3, max(nblk)), -1, np.int32)
    off = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm0[off:off + n]
        off += n
    tk, tv = _rand_tokens(rng, 3, max(nblk) * bs, Hkv, D)
    tk = [np.asarray(oracle.encode_rows(x, "f32", "f32", 1.0)) for x in tk]
    kc, vc = _store(tk, tv, tables, lens, bs=bs, NB=NB)
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    kw = dict(scale=1 / math.sqrt(D), bs=bs, q_dtype="f32", kv_dtype="f32")
    base = oracle.decode(q, kc, vc, tables, np.array(lens), **kw)
    pi = rng.permutation(NB)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = oracle.decode(q, kc2, vc2, t2, np.array(lens), **kw)
    np.testing.assert_array_equal(moved, base)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
def test_one_token_context_returns_v(kv_dtype):
    rng = np.random.default_rng(7)
    Hkv, Hq, D, bs = 2, 8, 128, 32 if kv_dtype == "fp8" else 16
    src = "f32" if kv_dtype == "f32" else "bf16"
    k = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    if src == "bf16":
        k = torch.from_numpy(k).bfloat16().view(torch.int16).numpy().view(np.uint16)
        v = torch.from_numpy(v).bfloat16().view(torch.int16).numpy().view(np.uint16)
    kc = oracle.new_cache(4, Hkv, bs, D, kv_dtype)
    vc = oracle.new_cache(4, Hkv, bs, D, kv_dtype)
    oracle.reshape_and_cache(kc, vc, k, v, np.array([2 * bs]), bs=bs, src_dtype=src,
                             kv_dtype=kv_dtype, k_scale=0.01, v_scale=0.02)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, np.array([[2]]), np.array([1]), scale=0.1, bs=bs, q_dtype="f32",
                        kv_dtype=kv_dtype, k_scale=0.01, v_scale=0.02)
    vstored = oracle.gather_kv(vc, [2], 1, "v", bs=bs, kv_dtype=kv_dtype, scale=0.02)[0]
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_array_equal(out[0, h], vstored[h // G])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(8)
    Hkv, Hq, D, bs, L = 2, 4, 64, 16, 77
    row = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    tk = [np.repeat(row, 80, axis=0)]
    tv = [rng.standard_normal((80, Hkv, D)).astype(np.float32)]
    table = rng.permutation(9)[:5].astype(np.int32)
    kc, vc = _store(tk, tv, table[None], [L], bs=bs, NB=9)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, table[None], np.array([L]), scale=0.3, bs=bs, q_dtype="f32",
                        kv_dtype="f32")
    mean = tv[0][:L].astype(np.float64).mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], mean[h // 2], rtol=0, atol=1e-13)


def test_dominant_key_decodes_to_its_value():
    """When one key's scaled score (log2 of its softmax weight) exceeds every other key's by at
    least 29, the others together carry less than L * 2^-29 of the weight, so the output is that
    key's value to within that fraction of the largest value.  The steered spike case puts one
    key 60 above a level in [-2, 2] and a second one 30 above it."""
    import workloads
    base = workloads.decode_case("dominant", 21, Hq=4, Hkv=2, D=64, bs=16, lens=[2100],
                                 kv_dtype="f32", std=1.0, pool="scattered")
    c = workloads.steer_scores(base, 9, "spike")
    kc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, "f32")
    vc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, "f32")
    oracle.reshape_and_cache(kc, vc, c.pool_k, c.pool_v, np.arange(c.NB * c.bs), bs=c.bs,
                             src_dtype="f32", kv_dtype="f32")
    oracle.reshape_and_cache(kc, vc, c.new_k, c.new_v, c.new_slots, bs=c.bs, src_dtype="f32",
                             kv_dtype="f32")
    out = oracle.decode(c.q, kc, vc, c.block_tables, c.context_lens, scale=c.scale, bs=c.bs,
                        q_dtype="f32", kv_dtype="f32")
    t = (3 * 2099) // 4
    slot = int(c.block_tables[0, t // c.bs]) * c.bs + t % c.bs
    v_top = c.pool_v[slot].astype(np.float64)  # [Hkv, D]
    tt = np.arange(2099)
    live = c.block_tables[0, tt // c.bs].astype(np.int64) * c.bs + tt % c.bs
    vmax = max(np.abs(c.pool_v[live]).max(), np.abs(c.new_v).max())
    bound = 2100 * 2.0 ** -29 * vmax
    for h in range(c.Hq):
        np.testing.assert_allclose(out[0, h], v_top[h // c.G], rtol=0, atol=bound)


def _brute_decode(q, K, V, scale):
    """Attention with explicit Python loops and math.exp (q [Hq, D], K/V [L, Hkv, D])."""
    Hq, D = q.shape
    L, Hkv = K.shape[:2]
    G = Hq // Hkv
    out = [[0.0] * D for _ in range(Hq)]
    for h in range(Hq):
        g = h // G
        s = [scale * sum(float(q[h, d]) * float(K[t, g, d]) for d in range(D)) for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for d in range(D):
            out[h][d] = sum(w[t] * float(V[t, g, d]) for t in range(L)) / z
    return np.array(out)


# ----------------------------------------------------------------------------- fp8 dequantisation
#
# infoisland, section 4 ("--kv-cache-dtype fp8"): the cache stores one e4m3fn code per element,
# and the per-tensor K and V scales turn a code back into a value as code value x scale.  The
# expected values below are written by hand from the code table (0x30 = 0.5, 0x38 = 1, 0x3C =
# 1.5, 0x40 = 2, 0x48 = 4, 0xB8 = -1, 0xC0 = -2, 0x01 = 2^-9) and the scales, not computed by
# the reference's own gather.


def _fp8_cache_with_rows(rows, kind, *, bs=32, D=64, NB=3, frame=1, fill=0x00):
    """An fp8 cache of NB frames, one kv head, whose frame `frame` holds token t's row of codes
    rows[t] (a length-D list, or one code for the whole row); other slots hold `fill`."""
    vals = np.full((NB, 1, bs, D), fill, dtype=np.uint8)
    for t, r in enumerate(rows):
        vals[frame, 0, t, :] = r
    return oracle.pack_tiles(vals, kind, "fp8").reshape(NB, 1, bs * D)


def test_fp8_one_token_output_is_code_value_times_v_scale():
    D = 64
    vrow = [0x3C, 0xC0, 0x30, 0x01] + [0x38] * (D - 4)
    kc = _fp8_cache_with_rows([[0x40] * D], "k", fill=0x7E)
    vc = _fp8_cache_with_rows([vrow], "v", fill=0x7E)
    q = np.random.default_rng(21).standard_normal((1, 2, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, np.array([[1]]), np.array([1]), scale=0.125, bs=32,
                        q_dtype="f32", kv_dtype="fp8", k_scale=3.0, v_scale=0.25)
    want = [0.375, -0.5, 0.125, 2.0 ** -11] + [0.25] * (D - 4)
    for h in range(2):
        assert out[0, h].tolist() == want


def _two_token_fp8_case():
    D = 64
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    kc = _fp8_cache_with_rows([[0x38] + [0x00] * (D - 1), [0x40] + [0x00] * (D - 1)], "k",
                              fill=0x7E)
    vc = _fp8_cache_with_rows([0x38, 0x48], "v", fill=0x7E)
    return q, kc, vc


def test_fp8_two_token_softmax_depends_on_k_scale():
    # k_scale 0.5: keys 1 and 2 score 0.5 and 1.0, so the second token weighs 1 / (1 + e^-0.5);
    # v_scale 0.125: values 1 and 4 become 0.125 and 0.5.
    q, kc, vc = _two_token_fp8_case()
    out = oracle.decode(q, kc, vc, np.array([[1]]), np.array([2]), scale=1.0, bs=32,
                        q_dtype="f32", kv_dtype="fp8", k_scale=0.5, v_scale=0.125)
    want = 0.125 + 0.375 / (1.0 + math.exp(-0.5))
    assert abs(want - 0.35842224920069548) < 1e-15
    np.testing.assert_allclose(out[0, 0], np.full(64, want), rtol=0, atol=1e-15)


def test_fp8_two_row_chunk_closed_form():
    # The same two tokens as one causal chunk of two rows (bicarait.com, "Architectural
    # Blueprint 3"): row 0 sees only the first token and returns its value 0.125; row 1 sees
    # both, as in the decode case above.
    q, kc, vc = _two_token_fp8_case()
    q2 = np.concatenate([q, q], axis=0)
    out = oracle.prefill_chunk(q2, kc, vc, np.array([[1]]), np.array([0, 2]), np.array([2]),
                               scale=1.0, bs=32, q_dtype="f32", kv_dtype="fp8", k_scale=0.5,
                               v_scale=0.125)
    assert out[0, 0].tolist() == [0.125] * 64
    np.testing.assert_allclose(out[1, 0], 0.125 + 0.375 / (1.0 + math.exp(-0.5)), rtol=0,
                               atol=1e-15)


def test_fp8_identical_keys_mean_of_values_times_v_scale():
    # Five tokens with the same key codes: every weight is 1/5, so the output is
    # 0.75 x mean(1, 2, 0.5, 1.5, -1) = 0.75 x 0.8 = 0.6 in every column.
    D = 64
    key = np.random.default_rng(22).integers(0, 0x7E, D).astype(np.uint8)
    kc = _fp8_cache_with_rows([key] * 5, "k", fill=0x7E)
    vc = _fp8_cache_with_rows([0x38, 0x40, 0x30, 0x3C, 0xB8], "v", fill=0x7E)
    q = np.random.default_rng(23).standard_normal((1, 4, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, np.array([[1]]), np.array([5]), scale=0.3, bs=32,
                        q_dtype="f32", kv_dtype="fp8", k_scale=2.0, v_scale=0.75)
    np.testing.assert_allclose(out[0], np.full((4, D), 0.6), rtol=0, atol=1e-15)


def test_fp8_store_then_gather_round_trips_with_distinct_scales():
    # Rows stored with k_scale and v_scale (x / scale, rounded to a code) and read back (code x
    # scale) come back within the e4m3fn rounding bound: 2^-4 relative for normal codes, half
    # the subnormal step 2^-10 times the scale absolute.
    rng = np.random.default_rng(24)
    Hkv, D, bs, L = 2, 64, 32, 40
    k = (rng.standard_normal((L, Hkv, D)) * 3.0).astype(np.float32)
    v = (rng.standard_normal((L, Hkv, D)) * 0.02).astype(np.float32)
    ks, vs = float(np.abs(k).max() / 448), float(np.abs(v).max() / 448)
    assert vs < ks / 50
    kc = oracle.new_cache(4, Hkv, bs, D, "fp8")
    vc = oracle.new_cache(4, Hkv, bs, D, "fp8")
    table = np.array([3, 0], dtype=np.int32)
    oracle.reshape_and_cache(kc, vc, k, v, oracle.slot_of(table, np.arange(L), bs), bs=bs,
                             src_dtype="f32", kv_dtype="fp8", k_scale=ks, v_scale=vs)
    for x, c, kind, s in ((k, kc, "k", ks), (v, vc, "v", vs)):
        back = oracle.gather_kv(c, table, L, kind, bs=bs, kv_dtype="fp8", scale=s)
        x64 = x.astype(np.float64)
        bound = np.abs(x64) * 2.0 ** -4 + 2.0 ** -10 * s
        assert np.all(np.abs(back - x64) <= bound)


def test_brute_force_every_injective_table():
    rng = np.random.default_rng(9)
    Hkv, Hq, D, bs, L, NB = 1, 2, 16, 16, 37, 5  # 3 blocks into a 5-frame pool: 60 tables
    tk, tv = _rand_tokens(rng, 1, 3 * bs, Hkv, D)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    want = _brute_decode(q[0], tk[0][:L], tv[0][:L], 0.25)
    n = 0
    for table in itertools.permutations(range(NB), 3):
        t = np.array(table, dtype=np.int32)[None]
        kc, vc = _store(tk, tv, t, [L], bs=bs, NB=NB)
        out = oracle.decode(q, kc, vc, t, np.array([L]), scale=0.25, bs=bs, q_dtype="f32",
                            kv_dtype="f32")
        np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)
        n += 1
    assert n == 60


def test_poison_outside_context_is_never_read():
    rng = np.random.default_rng(10)
    Hkv, Hq, D, bs, L = 2, 4, 64, 16, 21
    tk, tv = _rand_tokens(rng, 1, 2 * bs, Hkv, D)
    tk[0][L:] = 30.0
    tv[0][L:] = 1000.0
    table = np.array([[3, 1]], dtype=np.int32)
    kc, vc = _store(tk, tv, table, [2 * bs], bs=bs, NB=6)  # tail slots hold poison
    kc[[0, 2, 4, 5]] = np.float32(30.0)
    vc[[0, 2, 4, 5]] = np.float32(1000.0)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, table, np.array([L]), scale=0.125, bs=bs, q_dtype="f32",
                        kv_dtype="f32")
    ref = _sdpa(q[0][:, None, :].astype(np.float64), tk[0][:L].astype(np.float64),
                tv[0][:L].astype(np.float64), 0.125)[:, 0]
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- cache writes


def test_reshape_and_cache_skips_negative_slots_and_round_trips():
    rng = np.random.default_rng(11)
    Hkv, D, bs, NB = 2, 128, 16, 4
    k = torch.from_numpy(rng.standard_normal((6, Hkv, D)).astype(np.float32)).bfloat16()
    k = k.view(torch.int16).numpy().view(np.uint16)
    v = k[::-1].copy()
    slots = np.array([5, -1, 17, 63, -7, 0], dtype=np.int64)
    kc = oracle.new_cache(NB, Hkv, bs, D, "bf16")
    vc = oracle.new_cache(NB, Hkv, bs, D, "bf16")
    oracle.reshape_and_cache(kc, vc, k, v, slots, bs=bs, src_dtype="bf16", kv_dtype="bf16")
    kv = oracle.unpack_tiles(kc, "k", "bf16", bs, D)  # [NB, Hkv, bs, D]
    vv = oracle.unpack_tiles(vc, "v", "bf16", bs, D)
    written = np.zeros((NB, bs), bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written[s // bs, s % bs] = True
        np.testing.assert_array_equal(kv[s // bs, :, s % bs], k[i])
        np.testing.assert_array_equal(vv[s // bs, :, s % bs], v[i])
    assert np.all(kv.transpose(0, 2, 1, 3)[~written] == 0)


def test_reshape_and_cache_fp8_uses_scaled_rne():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((3, 1, 128)) * 3).astype(np.float32)
    xb = torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16)
    kc = oracle.new_cache(2, 1, 32, 128, "fp8")
    vc = oracle.new_cache(2, 1, 32, 128, "fp8")
    ks = np.float32(3.5) / np.float32(448)
    oracle.reshape_and_cache(kc, vc, xb, xb, np.array([0, 33, 63]), bs=32, src_dtype="bf16",
                             kv_dtype="fp8", k_scale=float(ks), v_scale=2.0)
    xf = oracle.bf16_bits_to_f64(xb).astype(np.float32)
    kv = oracle.unpack_tiles(kc, "k", "fp8", 32, 128)
    vv = oracle.unpack_tiles(vc, "v", "fp8", 32, 128)
    for i, s in enumerate([0, 33, 63]):
        want_k = torch.from_numpy(np.clip(xf[i] / ks, -448, 448)).to(torch.float8_e4m3fn)
        np.testing.assert_array_equal(kv[s // 32, :, s % 32], want_k.view(torch.uint8).numpy())
        want_v = torch.from_numpy(xf[i] / np.float32(2.0)).to(torch.float8_e4m3fn)
        np.testing.assert_array_equal(vv[s // 32, :, s % 32], want_v.view(torch.uint8).numpy())


def test_copy_blocks_shared_equals_private_copy():
    rng = np.random.default_rng(13)
    Hkv, Hq, D, bs, NB = 2, 4, 64, 16, 8
    kc = rng.standard_normal((NB, Hkv, bs * D)).astype(np.float32)
    vc = rng.standard_normal((NB, Hkv, bs * D)).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    kw = dict(scale=0.2, bs=bs, q_dtype="f32", kv_dtype="f32")
    shared = oracle.decode(q, kc, vc, np.array([[1, 4]]), np.array([29]), **kw)
    oracle.copy_blocks(kc, vc, [[4, 6], [1, 7]])
    np.testing.assert_array_equal(kc[6], kc[4])
    np.testing.assert_array_equal(vc[7], vc[1])
    private = oracle.decode(q, kc, vc, np.array([[7, 6]]), np.array([29]), **kw)
    np.testing.assert_array_equal(private, shared)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, vc, [[1, 2], [3, 2]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, vc, [[1, 2], [2, 3]])


# ----------------------------------------------------------------------------- prefill chunks


def _chunk_setup(rng, L, Hkv=2, Hq=8, D=64, bs=16, NB=None):
    nblk = -(-L // bs)
    NB = NB or nblk + 3
    table = rng.permutation(NB)[:nblk].astype(np.int32)[None]
    tk, tv = _rand_tokens(rng, 1, nblk * bs, Hkv, D)
    kc, vc = _store(tk, tv, table, [L], bs=bs, NB=NB)
    return table, tk[0], tv[0], kc, vc


def test_one_row_chunk_equals_decode():
    rng = np.random.default_rng(14)
    L, Hq, D = 45, 8, 64
    table, tk, tv, kc, vc = _chunk_setup(rng, L)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    kw = dict(scale=0.125, bs=16, q_dtype="f32", kv_dtype="f32")
    chunk = oracle.prefill_chunk(q, kc, vc, table, np.array([0, 1]), np.array([L]), **kw)
    dec = oracle.decode(q, kc, vc, table, np.array([L]), **kw)
    np.testing.assert_array_equal(chunk[0], dec[0])


def test_chunk_from_position_zero_is_causal_sdpa():
    rng = np.random.default_rng(15)
    L, Hq, D = 50, 8, 64
    table = np.arange(4, dtype=np.int32)[None]
    tk, tv = _rand_tokens(rng, 1, 64, 2, D)
    kc, vc = _store(tk, tv, table, [L], bs=16, NB=4)
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    out = oracle.prefill_chunk(q, kc, vc, table, np.array([0, L]), np.array([L]), scale=0.125,
                               bs=16, q_dtype="f32", kv_dtype="f32")
    ref = _sdpa(q.transpose(1, 0, 2).astype(np.float64), tk[0][:L].astype(np.float64),
                tv[0][:L].astype(np.float64), 0.125, causal=True)
    np.testing.assert_allclose(out, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_two_chunks_of_n_equal_one_chunk_of_2n():
    rng = np.random.default_rng(16)
    L, n, Hq, D = 90, 20, 8, 64
    table, tk, tv, kc, vc = _chunk_setup(rng, L)
    q = rng.standard_normal((2 * n, Hq, D)).astype(np.float32)
    kw = dict(scale=0.125, bs=16, q_dtype="f32", kv_dtype="f32")
    whole = oracle.prefill_chunk(q, kc, vc, table, np.array([0, 2 * n]), np.array([L]), **kw)
    two = oracle.prefill_chunk(q, kc, vc, np.concatenate([table, table]), np.array([0, n, 2 * n]),
                               np.array([L - n, L]), **kw)
    np.testing.assert_array_equal(two, whole)


def test_mixed_step_equals_decodes_and_chunks_alone():
    import workloads

    c = workloads.chunk_case("mix", 17, Hq=8, Hkv=2, D=64, bs=16,
                             chunks=[(20, 70), (16, 16), (5, 40)], decode_lens=[1, 5, 33, 48],
                             kv_dtype="bf16", std=0.7071)
    kw = dict(bs=c.bs, src_dtype=c.src_dtype, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
              v_scale=c.v_scale)
    kc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype)
    vc = oracle.new_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype)
    oracle.reshape_and_cache(kc, vc, c.pool_k, c.pool_v, c.pool_slots, **kw)
    oracle.reshape_and_cache(kc, vc, c.new_k, c.new_v, c.new_slots, **kw)
    m = workloads.mixed_batch(c)
    akw = dict(scale=c.scale, bs=c.bs, q_dtype=c.q_dtype, kv_dtype=c.kv_dtype,
               k_scale=c.k_scale, v_scale=c.v_scale)
    mixed = oracle.mixed_attention(m.q, kc, vc, m.block_tables, m.query_start_loc,
                                   m.context_lens, m.num_decodes, **akw)
    dec = oracle.decode(c.q, kc, vc, c.block_tables, c.context_lens, **akw)
    ch = c.chunk
    chunk = oracle.prefill_chunk(ch.q, kc, vc, ch.block_tables, ch.query_start_loc,
                                 ch.context_lens, **akw)
    assert mixed.shape[0] == c.B + ch.q.shape[0]
    np.testing.assert_array_equal(mixed[:c.B], dec)
    np.testing.assert_array_equal(mixed[c.B:], chunk)
    bad = m.query_start_loc.copy()
    bad[1] = 2
    with pytest.raises(ValueError):
        oracle.mixed_attention(m.q, kc, vc, m.block_tables, bad, m.context_lens, m.num_decodes,
                               **akw)
