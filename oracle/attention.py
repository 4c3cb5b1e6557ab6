"""Core attention over the selected FP4 entries and the sliding window.

Follows [atlas] section 3.2: one main Q attends the sparse main-KV branch and
the uncompressed window KV, and the two are merged (heterogeneous KV figure);
the main KV is the 512-wide latent shared across heads ([stamatios], "CSA2:
compressão em três dimensões") stored as FP4 and dequantised just before
attention ([newsaint] section 4).  Reuse layers run the same computation with a
new main Q and the inherited index set ([atlas] section 3.2 mode table).

Readings (also in the design notes):
* MLA-absorbed form: key_j = [latent_j (512) || rope_j (64)], value_j =
  latent_j; logits l_j = scale * (q_lat . key_j[:512] + q_rope . key_j[512:]);
* one softmax over the union of the sparse entries and the window rows
  [c, n); the output per head is the 512-wide latent mix;
* window rows come from a separate bf16 buffer of latent || rope values.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_kv
from .formats import bf16_to_f64


def gather_entries(codes_rows, scales_rows, rope_rows_bits, swa_rows_bits):
    """Build the float64 key matrix [E, 576] from the sparse rows (FP4 codes,
    E4M3 scales, bf16 rope) followed by the window rows (bf16 [w, 576])."""
    parts = []
    if len(codes_rows):
        lat = decode_kv(codes_rows, scales_rows)
        parts.append(np.concatenate([lat, bf16_to_f64(rope_rows_bits)], axis=1))
    if len(swa_rows_bits):
        parts.append(bf16_to_f64(swa_rows_bits))
    if not parts:
        return np.zeros((0, 576))
    return np.concatenate(parts, axis=0)


def attend(q_lat_bits, q_rope_bits, scale: float, keys: np.ndarray):
    """q_lat [H, 512], q_rope [H, 64] bf16 bits; keys float64 [E, 576].
    Returns (out float64 [H, 512], lse float64 [H]); E = 0 gives out = 0 and
    lse = -inf."""
    q = np.concatenate([bf16_to_f64(q_lat_bits), bf16_to_f64(q_rope_bits)], axis=1)
    H = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((H, 512)), np.full(H, -np.inf)
    logits = float(scale) * (q @ keys.T)              # [H, E]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e / l) @ keys[:, :512]
    return out, (m + np.log(l))[:, 0]
