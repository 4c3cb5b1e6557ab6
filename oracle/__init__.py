"""CPU oracle for the CSA2 decode path (test infrastructure only).

A plain, slow, float64 NumPy statement of what the decode path computes:
FP4 main-KV encode/decode (and the same codec at other widths for the FP4
indexer variant), the Full-mode indexer (scores, block-of-8 maxima,
the Top-P block pool), Reindex inside the pool, and the joint sparse + window
attention with one softmax.  Each function cites the page passage it follows.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library, and the GPU
library never calls it.

Sources cited (web pages about DeepSeek-V4.1-Flash):
  [newsaint]  "DeepSeek-V4.1-Flash 2026: Arsitektur Causal Encoder-Decoder
               (CED), Compressed Sparse Attention 2 (CSA2), FP4 KV Caching,
               dan SWA Bounded Replay untuk 1M Context Window"
  [stamatios] "DeepSeek-V4.1 Flash comprime cache KV para 890 bytes por token"
  [atlas]     "DeepSeek-V4.1-Flash 梗概" (deepseek-mechanism-atlas)
  [akhunji]   "DeepSeek-V4.1-Flash Architecture: Causal Encoder-Decoder (CED),
               890-Byte KV Cache, Engram Memory, and CSA2"

Parity status: every function here is pinned by tests that do not re-derive
it (closed forms, library special cases, brute force, invariants).  The pages
print no worked numeric example, so no pin is a page-printed value except the
format constants (E2M1 levels, the E4M3 maximum, group and block sizes).
"""
from .formats import (E2M1_LEVELS, bf16_to_f64, e4m3_decode, e4m3_encode_rne,
                      e2m1_encode_rne)
from .codec import encode_kv, decode_kv, encode_fp4, decode_fp4, BYTES_CODES, BYTES_SCALES, GROUP
from .indexer import (candidates, index_scores, block_scores, select_pool,
                      pool_positions, reindex, index_full, rank_order, decode_rows,
                      take_rows, n_rows)
from .attention import attend, gather_entries

__all__ = [
    "E2M1_LEVELS", "bf16_to_f64", "e4m3_decode", "e4m3_encode_rne",
    "e2m1_encode_rne", "encode_kv", "decode_kv", "encode_fp4", "decode_fp4",
    "BYTES_CODES", "BYTES_SCALES",
    "GROUP", "candidates", "index_scores", "block_scores", "select_pool",
    "pool_positions", "reindex", "index_full", "rank_order", "decode_rows",
    "take_rows", "n_rows", "attend",
    "gather_entries",
]
