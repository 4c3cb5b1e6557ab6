"""Full-mode hierarchical indexer and Reindex.

Follows [atlas] section 3.2: the mode table (Full scores everything and takes
a new Top-K; Reindex re-scores with this layer's indexer query and reuses the
indexer keys of the last Full layer) and the hierarchical sparse indexer
paragraph (blocks of 8 positions, the Top-2048 blocks, about 16,384 positions,
form the candidate pool; later Reindex layers score only inside the pool and
keep the Top-512).  [newsaint] section 3 states the O(N) Full scan over every
causally visible position and the constant-size pool for deeper layers; its
section 8 simulation gathers only the pool's keys for re-indexing.
[atlas] section 3.2 (heterogeneous KV figure) routes the indexer and Top-K to
the sparse branch only, so the sliding window is never a candidate.

Readings where the pages are silent (also listed in the design notes):
* score of position p:  s_p = sum_h w_h * max(0, q_h . k_p), with one fp8
  key per position shared by all indexer heads and fp32 per-head weights;
* candidates are p in [0, c), c = max(0, n - W), for a query seeing [0, n);
* blocks are aligned at multiples of 8; block score = max over its candidate
  positions; the partial block at c takes its max over p < c only;
* order is (score descending, position or block ascending): ties go to the
  lower index; outputs are ascending; fewer candidates than capacity -> all.

FP4 indexer variant ([newsaint] section 4: DeepSeek-V4 trained the indexer's
query and key with FP4 QAT): every function below also takes its queries and
keys as FP4 pairs (codes [.., d / 2], scales [.., d / 16]) in the row codec of
`codec.encode_fp4`; the scores are the same formula over the decoded values.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_fp4
from .formats import e4m3_decode

BLOCK = 8


def candidates(n: int, W: int) -> int:
    """Number of sparse candidates c = max(0, n - W)."""
    return max(0, int(n) - int(W))


def decode_rows(x) -> np.ndarray:
    """Indexer rows as float64: fp8 E4M3FN bytes [.., d], or an FP4 pair
    (codes [.., d / 2], scales [.., d / 16]) decoded by the FP4 codec."""
    if isinstance(x, tuple):
        codes, scales = (np.asarray(v) for v in x)
        lead = codes.shape[:-1]
        v = decode_fp4(codes.reshape(-1, codes.shape[-1]), scales.reshape(-1, scales.shape[-1]))
        return v.reshape(*lead, v.shape[-1])
    return e4m3_decode(x)


def take_rows(x, idx):
    """Rows `idx` of an fp8 row array or of both planes of an FP4 pair."""
    if isinstance(x, tuple):
        return tuple(np.asarray(v)[idx] for v in x)
    return np.asarray(x)[idx]


def n_rows(x) -> int:
    return len(x[0]) if isinstance(x, tuple) else len(x)


def index_scores(q_codes, w: np.ndarray, k_codes) -> np.ndarray:
    """s_p = sum_h w_h * max(0, sum_i q[h,i] k[p,i]) in float64.

    q_codes [H_i, d], w float32 [H_i], k_codes [c, d]: fp8 e4m3fn bytes, or
    FP4 pairs (see `decode_rows`).  The inner sums are exact in float64.
    fp8: products carry at most 8 significant bits and are multiples of
    2^-18 below 2^18, so d <= 128 of them span under 53 bits.  FP4: a value
    (E2M1 level x E4M3 scale) is a multiple of 2^-10 below 2688, so products
    are multiples of 2^-20 below 2^23, and 128 of them span under 51 bits.
    """
    q = decode_rows(q_codes)                        # [H_i, d]
    k = decode_rows(k_codes)                        # [c, d]
    dots = k @ q.T                                   # [c, H_i]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def block_scores(s: np.ndarray) -> np.ndarray:
    """b_j = max of s over [8j, min(8j + 8, c)), j < ceil(c / 8)."""
    c = len(s)
    nb = -(-c // BLOCK)
    pad = np.full(nb * BLOCK, -np.inf)
    pad[:c] = s
    return pad.reshape(nb, BLOCK).max(axis=1) if nb else np.zeros(0)


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Indices sorted by (score descending, index ascending)."""
    idx = np.arange(len(scores))
    return np.lexsort((idx, -np.asarray(scores, dtype=np.float64)))


def select_pool(b: np.ndarray, P: int) -> np.ndarray:
    """The min(P, nb) best blocks, ascending block ids (int64)."""
    return np.sort(rank_order(b)[: min(P, len(b))])


def pool_positions(pool: np.ndarray, c: int) -> np.ndarray:
    """Candidate positions of the pool blocks (ascending), p < c only."""
    pos = (np.asarray(pool, dtype=np.int64)[:, None] * BLOCK + np.arange(BLOCK)).reshape(-1)
    return pos[pos < c]


def reindex(q_codes, w, k_codes_all, pool, c: int, K: int):
    """Reindex: score only the pool's candidate positions with (q', w') and
    keep the Top-min(K, |R|) by (score desc, position asc).

    k_codes_all: the query's key rows indexed by position (at least c rows).
    Returns (ascending positions int64, scores of all pool positions, R)."""
    if n_rows(k_codes_all) < c:
        raise ValueError("key rows must cover every candidate position")
    R = pool_positions(pool, c)
    s = index_scores(q_codes, w, take_rows(k_codes_all, R)) if len(R) else np.zeros(0)
    keep = np.sort(R[rank_order(s)[: min(K, len(R))]])
    return keep, s, R


def index_full(q_codes, w, k_codes_all, n: int, W: int, P: int):
    """Full mode: scores over every candidate, block maxima, Top-P blocks.
    Returns (pool ascending int64, block scores float64, position scores)."""
    c = candidates(n, W)
    if n_rows(k_codes_all) < c:
        raise ValueError("key rows must cover every candidate position")
    s = index_scores(q_codes, w, take_rows(k_codes_all, slice(0, c))) if c else np.zeros(0)
    b = block_scores(s)
    return select_pool(b, P), b, s
