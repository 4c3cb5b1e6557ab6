"""Number formats used by the decode path, defined bit by bit.

* bf16: the upper 16 bits of an IEEE binary32; every value is exact in f64.
* OCP FP8 E4M3FN ("E4M3", maximum 448 as stated beside the quantiser in
  [newsaint] section 8 and named as the FP4 scale format in [atlas] section
  3.2): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds
  subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; there is no infinity.
* E2M1 (FP4): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, the level list printed
  in the FP4Quantizer of [newsaint] section 8; magnitude code = index in that
  list, sign in bit 3.
"""
from __future__ import annotations

import numpy as np

E2M1_LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16/int16 array) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):                 # NaN payloads
        return b.view(np.float32).astype(np.float64)


def e4m3_decode(code) -> np.ndarray:
    """OCP E4M3FN byte -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# The 127 finite non-negative E4M3FN values in increasing order; code == index.
_E4M3_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode_rne(t) -> np.ndarray:
    """Round non-negative finite values in [0, 448] to E4M3FN, nearest value,
    ties to the even code (even mantissa).  Returns uint8 codes 0x00..0x7E."""
    t = np.asarray(t, dtype=np.float64)
    if np.any(~np.isfinite(t)) or np.any(t < 0) or np.any(t > 448.0):
        raise ValueError("e4m3_encode_rne expects values in [0, 448]")
    hi = np.searchsorted(_E4M3_POS, t, side="left")          # first value >= t
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _E4M3_POS[lo], _E4M3_POS[hi]
    exact = vhi == t
    dlo, dhi = t - vlo, vhi - t                                # exact in f64
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    return code.astype(np.uint8)


def e2m1_encode_rne(r) -> np.ndarray:
    """Non-negative ratio r -> E2M1 magnitude code 0..7: the nearest level of
    E2M1_LEVELS, ties to the even code, saturating at 6 for r > 6."""
    r = np.asarray(r, dtype=np.float64)
    if np.any(r < 0) or np.any(np.isnan(r)):
        raise ValueError("e2m1_encode_rne expects non-negative ratios")
    d = np.abs(r[..., None] - E2M1_LEVELS)                    # distance to each level
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                          # one or two nearest levels
    codes = np.arange(8)
    even_tie = cand & (codes % 2 == 0)
    has_even = even_tie.any(axis=-1, keepdims=True)
    choose = np.where(has_even & (cand.sum(-1, keepdims=True) > 1), even_tie, cand)
    code = np.argmax(choose, axis=-1)
    return np.where(r > 6.0, 7, code).astype(np.uint8)          # saturate
