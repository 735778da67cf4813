"""Planted mistakes in the CPU reference must fail its pins.

Each case patches one piece of oracle/ (on the CPU only) with a plausible bug
and checks that at least one pin from test_oracle.py then fails.
"""

import numpy as np
import pytest

import oracle.layout as L
import oracle.numerics as N
import oracle.paged_attention as P
from tests import test_oracle as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError, FloatingPointError):
        return True
    return False


def _slot_off_by_one(table_row, positions, bs):
    positions = np.asarray(positions, dtype=np.int64)
    return np.asarray(table_row, dtype=np.int64)[positions // bs] * bs + (positions + 1) % bs


def _gather_ignores_table(cache, table_row, Lq, kind, *, bs, kv_dtype, scale=1.0):
    return _ORIG_GATHER(cache, np.arange(len(table_row)), Lq, kind, bs=bs, kv_dtype=kv_dtype,
                        scale=scale)


def _softmax_max_normalised(qrows, K, V, scale):
    s = scale * (K @ qrows.T)
    p = np.exp(s - s.max(axis=0, keepdims=True))
    return (p.T @ V) / p.max(axis=0)[:, None]


def _softmax_drops_last_key(qrows, K, V, scale):
    return _ORIG_ATTEND(qrows, K[:-1] if len(K) > 1 else K, V[:-1] if len(V) > 1 else V, scale)


def _scale_after_softmax(qrows, K, V, scale):
    return scale * _ORIG_ATTEND(qrows, K, V, 1.0)


def _bf16_wrong_shift(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    out = _ORIG_ENC(y)
    t = N.e4m3fn_table()
    fin = (out & 0x7F) < 0x7E
    up = (out + 1).astype(np.uint8)
    mid = np.abs((t[out & 0x7F] + t[(out & 0x7F) + fin]) / 2) == np.abs(y.astype(np.float64))
    return np.where(mid & fin, up, out).astype(np.uint8)


def _positions_transposed(kind, bs, D, dtype):
    pos = _ORIG_POS(kind, bs, D, dtype)
    return pos.T.reshape(bs, D) if kind == "v" else pos


def _dequant_divides(cache, table_row, Lq, kind, *, bs, kv_dtype, scale=1.0):
    vals = _ORIG_GATHER(cache, table_row, Lq, kind, bs=bs, kv_dtype=kv_dtype, scale=1.0)
    return vals / float(np.float32(scale)) if kv_dtype == "fp8" else vals


def _dequant_twice(cache, table_row, Lq, kind, *, bs, kv_dtype, scale=1.0):
    vals = _ORIG_GATHER(cache, table_row, Lq, kind, bs=bs, kv_dtype=kv_dtype, scale=scale)
    return vals * float(np.float32(scale)) if kv_dtype == "fp8" else vals


def _decode_swaps_scales(*args, k_scale=1.0, v_scale=1.0, **kw):
    return _ORIG_DECODE(*args, k_scale=v_scale, v_scale=k_scale, **kw)


def _chunk_swaps_scales(*args, k_scale=1.0, v_scale=1.0, **kw):
    return _ORIG_CHUNK(*args, k_scale=v_scale, v_scale=k_scale, **kw)


_ORIG_GATHER = P.gather_kv
_ORIG_DECODE = P.decode
_ORIG_CHUNK = P.prefill_chunk
_ORIG_ENC = N.e4m3fn_encode
_ORIG_ATTEND = P._softmax_attend
_ORIG_POS = L.tile_positions

MUTANTS = [
    ("slot offset off by one", P, "slot_of", _slot_off_by_one,
     [pins.test_slot_of_follows_the_block_split_rule]),
    ("gather ignores the block table", P, "gather_kv", _gather_ignores_table,
     [lambda: pins.test_diagram_block_tables("block_table_codebumble")]),
    ("softmax normalised by its max", P, "_softmax_attend", _softmax_max_normalised,
     [lambda: pins.test_identity_table_equals_textbook_attention(4, 2)]),
    ("last key dropped", P, "_softmax_attend", _softmax_drops_last_key,
     [lambda: pins.test_identity_table_equals_textbook_attention(4, 2),
      pins.test_chunk_from_position_zero_is_causal_sdpa]),
    ("scale applied after softmax", P, "_softmax_attend", _scale_after_softmax,
     [lambda: pins.test_identity_table_equals_textbook_attention(8, 8)]),
    ("bf16 decoded with the wrong shift", P, "bf16_bits_to_f64", _bf16_wrong_shift,
     [pins.test_bf16_decode_closed_form_and_torch]),
    ("fp8 ties rounded away from even", N, "e4m3fn_encode", _encode_ties_away,
     [pins.test_e4m3fn_encode_ties_saturation_nan]),
    ("V tile layout transposed", L, "tile_positions", _positions_transposed,
     [pins.test_tile_layout_hand_evaluated_entries]),
    ("fp8 codes divided by the scale", P, "gather_kv", _dequant_divides,
     [pins.test_fp8_one_token_output_is_code_value_times_v_scale,
      pins.test_fp8_store_then_gather_round_trips_with_distinct_scales]),
    ("fp8 scale applied twice", P, "gather_kv", _dequant_twice,
     [pins.test_fp8_two_token_softmax_depends_on_k_scale]),
    ("k_scale and v_scale swapped in decode", P, "decode", _decode_swaps_scales,
     [pins.test_fp8_one_token_output_is_code_value_times_v_scale]),
    ("k_scale and v_scale swapped in the chunk", P, "prefill_chunk", _chunk_swaps_scales,
     [pins.test_fp8_two_row_chunk_closed_form]),
]


@pytest.mark.parametrize("name,mod,attr,bad,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mod, attr, bad, checks):
    monkeypatch.setattr(mod, attr, bad)
    if mod is N:  # the tests call these through the package namespace
        import oracle
        monkeypatch.setattr(oracle, attr, bad)
    if mod is L:
        import oracle
        monkeypatch.setattr(pins, "tile_positions", bad)
        monkeypatch.setattr(oracle, attr, bad)
    if mod is P and attr in ("slot_of", "gather_kv", "decode", "prefill_chunk"):
        import oracle
        monkeypatch.setattr(oracle, attr, bad)
    if attr == "bf16_bits_to_f64":
        import oracle
        monkeypatch.setattr(oracle, attr, bad)
    assert any(_fails(c) for c in checks), f"planted mistake '{name}' went unnoticed"
