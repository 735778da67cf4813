"""Bit-level number formats for the oracle: bf16 and fp8 e4m3fn.

The pages ask only for an "fp8" KV cache that halves its footprint (infoisland,
section 4, the --kv-cache-dtype flag).  The format read here is OCP e4m3fn:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN at
the all-ones exponent with all-ones mantissa, largest finite magnitude 448.
Encoding is round-to-nearest-even of the fp32 quotient x / scale with
saturation to +-448; NaN stays NaN.  Both are readings of the page (it names
neither format nor rounding).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the bf16 bits are the high half of an fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (2.0 ** -6) * (m / 8.0)
    return s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 codes (float64; NaN at 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


_POS = _TABLE[:0x7F]  # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each fp32 value, ties to the even code, saturating at 448.

    Works by searching the sorted table of the 127 non-negative finite codes.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.where(np.signbit(y), 0x80, 0x00).astype(np.uint8)
    a_sat = np.minimum(a, 448.0)
    hi = np.searchsorted(_POS, a_sat, side="left")
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - _POS[lo]
    d_hi = _POS[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)
