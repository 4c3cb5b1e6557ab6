"""FP4 main-KV codec: E2M1 values with one E4M3 scale per 16 channels.

Follows [atlas] section 3.2 (FP4 main KV paragraph: E2M1, one E4M3 scale per
16 channels), [newsaint] section 4 (FP4 main KV, dequantised just before
attention) and the FP4Quantizer of [newsaint] section 8 (per-group absolute
maximum, scale = amax / 6 clamped to the E4M3 maximum 448, nearest E2M1
level), on the 512-wide latent shared across heads ([stamatios], "CSA2:
compressão em três dimensões").

Readings where the pages are silent or differ (each also listed in the design
notes):
* the scale is rounded to E4M3 with round-to-nearest-even after the 448 clamp
  (the quantiser on the page keeps it unrounded; a stored E4M3 scale must be
  rounded, and the plainest rounding is RNE);
* the E2M1 ratio |x|/s is rounded to nearest with ties to the even code (the
  page's argmin picks the smaller level on a tie);
* the sign bit is the sign of x, so a small negative value stores -0 (0x8);
  a group whose scale rounds to 0 stores all codes 0x0;
* two codes per byte, the even channel in the low nibble; the 32 scale bytes
  are stored apart from the 256 code bytes.

The same row codec at other widths (any multiple of 16 channels) encodes the
indexer's keys and queries in the FP4 indexer variant: [newsaint] section 4
states that DeepSeek-V4 already trained the indexer's query and key with FP4
QAT, before V4.1 extended FP4 to the main KV.  Reading: those rows use this
same E2M1 + one-E4M3-scale-per-16 format (the pages give no other FP4 layout
for them).

Group-32 variant of the main-KV codec: [akhunji] ("Microscopic FP4 (E2M1)
Cache Compression") pairs the E2M1 values with block-level FP8 scaling over
blocks of 32 elements.  Reading: the same rule (E4M3 scale = RNE of
min(amax / 6, 448) over the group, E2M1 RNE codes) with 32-channel groups,
16 scale bytes per 512-wide entry.  `encode_fp4(bits, group=32)` encodes it;
the decoders infer the group from the plane widths.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_LEVELS, bf16_to_f64, e2m1_encode_rne, e4m3_decode, e4m3_encode_rne

GROUP = 16          # channels per E4M3 scale
D_LATENT = 512
BYTES_CODES = D_LATENT // 2        # 256 code bytes per entry
BYTES_SCALES = D_LATENT // GROUP   # 32 scale bytes per entry


def encode_fp4(bits: np.ndarray, group: int = GROUP):
    """Encode bf16 rows [n, width] (uint16 bit patterns, width a multiple of
    the group) to (codes uint8 [n, width / 2], scales uint8 [n, width / group])."""
    lb = np.asarray(bits).astype(np.uint16)
    if group not in (16, 32) or lb.ndim != 2 or lb.shape[1] % group:
        raise ValueError("rows must be [n, width], width a multiple of the group (16 or 32)")
    n, width = lb.shape
    ng = width // group
    x = bf16_to_f64(lb).reshape(n, ng, group)
    neg = ((lb >> 15) & 1).astype(np.uint8).reshape(n, ng, group)
    amax = np.abs(x).max(axis=-1)                              # [n, groups]
    t = np.minimum(amax / 6.0, 448.0)
    scale_code = e4m3_encode_rne(t)                            # [n, groups]
    s = e4m3_decode(scale_code)
    zero = s == 0.0
    ratio = np.abs(x) / np.where(zero, 1.0, s)[..., None]
    mag = e2m1_encode_rne(ratio)                               # [n, groups, group]
    code = (neg << 3) | mag
    code = np.where(zero[..., None], 0, code).astype(np.uint8)
    code = code.reshape(n, width)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_code.astype(np.uint8)


def decode_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [n, width / 2], scales [n, width / group]) -> float64 [n, width]:
    value = (-1)^sign * E2M1 level * E4M3 scale (exact in float64).  The group
    (16 or 32 channels) is width / scales.shape[1]."""
    c = np.asarray(codes).astype(np.uint8)
    n, half = c.shape
    sc = np.asarray(scales)
    if sc.ndim != 2 or sc.shape[0] != n or sc.shape[1] == 0 or (2 * half) % sc.shape[1] \
            or (2 * half) // sc.shape[1] not in (16, 32):
        raise ValueError("scales must be [n, width / 16] or [n, width / 32]")
    group = (2 * half) // sc.shape[1]
    nib = np.empty((n, 2 * half), dtype=np.uint8)
    nib[:, 0::2] = c & 0xF
    nib[:, 1::2] = c >> 4
    sgn = np.where(nib >> 3, -1.0, 1.0)
    lev = E2M1_LEVELS[nib & 7]
    s = np.repeat(e4m3_decode(sc), group, axis=1)
    return sgn * lev * s


def encode_kv(latent_bits: np.ndarray, group: int = GROUP):
    """Encode bf16 latent rows [n, 512] (uint16 bit patterns) to
    (codes uint8 [n, 256], scales uint8 [n, 512 / group])."""
    lb = np.asarray(latent_bits).astype(np.uint16)
    if lb.ndim != 2 or lb.shape[1] != D_LATENT:
        raise ValueError("latent must be [n, 512]")
    return encode_fp4(lb, group)


def decode_kv(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [n, 256], scales [n, 32] or [n, 16]) -> float64 latent [n, 512]."""
    if np.asarray(codes).shape[1:] != (BYTES_CODES,):
        raise ValueError("codes must be [n, 256]")
    return decode_fp4(codes, scales)
