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
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode

BLOCK = 8


def candidates(n: int, W: int) -> int:
    """Number of sparse candidates c = max(0, n - W)."""
    return max(0, int(n) - int(W))


def index_scores(q_codes: np.ndarray, w: np.ndarray, k_codes: np.ndarray) -> np.ndarray:
    """s_p = sum_h w_h * max(0, sum_i q[h,i] k[p,i]) in float64.

    q_codes uint8 [H_i, d], w float32 [H_i], k_codes uint8 [c, d] (e4m3fn).
    The inner sums are exact in float64: fp8 products carry at most 8
    significant bits within [2^-18, 2^18], and d <= 128 of them fit 53 bits.
    """
    q = e4m3_decode(q_codes)                        # [H_i, d]
    k = e4m3_decode(k_codes)                        # [c, d]
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
    if len(k_codes_all) < c:
        raise ValueError("key rows must cover every candidate position")
    R = pool_positions(pool, c)
    s = index_scores(q_codes, w, np.asarray(k_codes_all)[R]) if len(R) else np.zeros(0)
    keep = np.sort(R[rank_order(s)[: min(K, len(R))]])
    return keep, s, R


def index_full(q_codes, w, k_codes_all, n: int, W: int, P: int):
    """Full mode: scores over every candidate, block maxima, Top-P blocks.
    Returns (pool ascending int64, block scores float64, position scores)."""
    c = candidates(n, W)
    if len(k_codes_all) < c:
        raise ValueError("key rows must cover every candidate position")
    s = index_scores(q_codes, w, np.asarray(k_codes_all)[:c]) if c else np.zeros(0)
    b = block_scores(s)
    return select_pool(b, P), b, s
