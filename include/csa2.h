/*
 * csa2.h -- C ABI of the CSA2 decode-path library for AMD Instinct MI355X
 * (gfx950): FP4 main-KV encode, Full-mode hierarchical indexer, Reindex, and
 * joint sparse + sliding-window attention.
 *
 * Sources (web pages about DeepSeek-V4.1-Flash):
 *   [atlas]     "DeepSeek-V4.1-Flash 梗概" (deepseek-mechanism-atlas), §3.2
 *               Compressed Sparse Attention 2: the Full / Reindex / Reuse mode
 *               table, the heterogeneous-KV figure, the hierarchical sparse
 *               indexer paragraph and the FP4 main-KV paragraph.
 *   [newsaint]  "DeepSeek-V4.1-Flash 2026: Arsitektur Causal Encoder-Decoder
 *               (CED), Compressed Sparse Attention 2 (CSA2), FP4 KV Caching,
 *               dan SWA Bounded Replay untuk 1M Context Window", §3 (indexer),
 *               §4 (FP4 main KV), §8 (FP4Quantizer, HierarchicalSparseIndexer).
 *   [stamatios] "DeepSeek-V4.1 Flash comprime cache KV para 890 bytes por
 *               token", "CSA2: compressão em três dimensões" (512-wide latent
 *               shared across heads; Full / Reindex / Reuse).
 *
 * Conventions for every call
 *   - Every array pointer is DEVICE memory owned by the caller.  The library
 *     never allocates or frees device memory; scratch comes from a caller
 *     workspace whose size the matching *_workspace_size call returns.
 *   - Calls validate their host-side arguments synchronously, then enqueue
 *     kernels on `stream` (a hipStream_t; NULL is the null stream) and return
 *     without waiting.  Outputs are ready when the stream reaches that point.
 *   - Per-query device data (seq_base, n_visible, swa_base, pool and top-k
 *     lists) are preconditions: they are not checked on the device.  Rows a
 *     query reads must exist in the caller's buffers.
 *   - bf16 arrays are passed as uint16_t bit patterns; fp8 arrays as uint8_t
 *     OCP E4M3FN bytes (maximum 448, the MI355X FP8 format).
 *   - FP4 rows (main KV, and the indexer rows of the *_fp4 calls) are two
 *     planes: codes, two E2M1 values per byte (the even channel in the low
 *     nibble, sign in bit 3 of each nibble), and scales, one E4M3FN byte per
 *     16 channels; value = E2M1 level x scale.
 *   - Non-finite inputs give undefined (but memory-safe) results.
 *   - Calls on different streams may run concurrently if their workspaces
 *     and outputs do not overlap.  The library's only mutable host state is
 *     per device and set once under a lock: the architecture check with the
 *     CU count it reads, and the largest dynamic-LDS size allowed for the
 *     pool kernel.
 *   - On error the call enqueues nothing and returns a status;
 *     csa2_last_error() gives a message for the calling thread.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 3

typedef enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,  /* null required pointer, bad size or dimension */
  CSA2_ERR_UNSUPPORTED = 2,  /* current device is not gfx950 */
  CSA2_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
  CSA2_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} csa2_status;

/* Problem dimensions.  Supported values:
 *   n_heads      H    main attention heads, a multiple of 8, 8..128
 *   d_latent          512 (the latent shared across heads; [stamatios])
 *   d_rope            64  (the bf16 RoPE key part)
 *   idx_heads    H_i  indexer heads, 1..64 (the scan keeps the query of all
 *                     heads resident in registers as MFMA operands, 32 VGPRs
 *                     per lane at 64 heads x 128 dims for fp8 rows and 64
 *                     for FP4 rows, beside the accumulators)
 *   idx_dim      d_i  indexer key / query width, 64 or 128
 *   block             8   (indexer block size; [atlas] §3.2)
 *   pool_blocks  P    blocks kept by the Full indexer, 1..2048
 *                     ([atlas] §3.2: Top-2048 blocks, about 16,384 positions)
 *   topk         K    positions kept by Reindex, 1..min(8*P, 2048)
 *                     ([atlas] §3.2: Top-512 inside the pool)
 *   swa          W    sliding-window rows, 0..1024
 *   kv_group          channels per main-KV FP4 scale: 16 ([atlas] §3.2), or
 *                     32 for the group-32 codec variant ([akhunji],
 *                     "Microscopic FP4 (E2M1) Cache Compression"); 0 means 16 */
typedef struct csa2_dims {
  int32_t n_heads;
  int32_t d_latent;
  int32_t d_rope;
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t block;
  int32_t pool_blocks;
  int32_t topk;
  int32_t swa;
  int32_t kv_group;
} csa2_dims;

/* A batch of decode queries.
 *   n_q             number of queries (>= 1).
 *   tokens_per_seq  g in 1..64: queries g*i .. g*i+g-1 belong to one
 *                   sequence (consecutive causal query tokens: a
 *                   speculative-verify step, or a prefill chunk scored by
 *                   the indexer against the cache) and MUST share seq_base; the
 *                   Full scan runs their workgroups for the same key range on
 *                   one XCD so the g key streams are served by one L2.
 *                   n_q must be a multiple of g.
 *   max_visible     host-side upper bound of every n_visible[i], at most
 *                   2^21; used only to size launch grids.
 *   seq_base        device int64 [n_q]: cache row of position 0 of the
 *                   query's sequence.  Position p lives at row seq_base + p
 *                   in idx_k, kv_codes, kv_scales and kv_rope.  In the
 *                   paged calls (csa2_pages) it is instead the offset of the
 *                   sequence's first page in the page table.
 *   n_visible       device int32 [n_q]: the query sees positions [0, n).
 * A query's sparse candidates are positions [0, c), c = max(0, n - W); the
 * window is [c, n) ([atlas] §3.2 heterogeneous KV: the indexer and Top-K
 * serve only the sparse branch). */
typedef struct csa2_queries {
  int32_t n_q;
  int32_t tokens_per_seq;
  int32_t max_visible;
  int32_t reserved;          /* must be 0 */
  const int64_t* seq_base;
  const int32_t* n_visible;
} csa2_queries;

/* Paged caches (serving integration: in [atlas] §3.2's mode figure a Full
 * layer writes each new token's main KV as decoding runs, and a serving cache
 * grows page by page; [akhunji], serving highlights).  In a call that
 * takes a csa2_pages, position p of query q's sequence lives at row
 *   table[seq_base[q] + p / page_size] * page_size + p % page_size
 * of every per-position plane the call reads (indexer keys and their scales;
 * kv_codes, kv_scales, kv_rope); seq_base[q] is then the offset in `table`
 * of the sequence's first page, not a row.  The window rows (swa_kv,
 * swa_base) are unchanged.
 *   table      device int32: physical page ids; entries for the pages that
 *              hold positions [0, n) of each query must be valid (< rows /
 *              page_size).  Caller-owned, read only.
 *   page_size  positions per page: a power of two in [16, 65536].
 *   reserved   must be 0.
 *   rows       rows of each plane the call reads (a multiple of page_size).
 *              The gathers address a plane with 32-bit byte offsets, so rows x
 *              the widest plane's row bytes (256 for kv_codes, d_i for fp8
 *              keys, d_i / 2 for FP4 key codes) must stay below 2^32 - 256:
 *              CSA2_ERR_INVALID_ARG otherwise. */
typedef struct csa2_pages {
  const int32_t* table;
  int32_t page_size;
  int32_t reserved;
  int64_t rows;
} csa2_pages;

/* ABI version of the loaded library (CSA2_ABI_VERSION). */
int32_t csa2_abi_version(void);

/* Static text for a status code. */
const char* csa2_status_string(csa2_status status);

/* Message describing the last error returned on the calling thread. */
const char* csa2_last_error(void);

/* FP4 main-KV encode ([atlas] §3.2 FP4 main KV; [newsaint] §4 and §8
 * FP4Quantizer).  For each of n entries and each group of 16 latent channels:
 *   amax = max |x|,  S = E4M3(round-to-nearest-even(min(amax / 6, 448))),
 *   s = value of S;  code_i = sign(x_i) << 3 | E2M1(|x_i| / s), the nearest
 *   E2M1 level with ties to the even code, saturating at 6;  s == 0 gives
 *   all codes 0.  Byte 8g+k of an entry's codes holds channel 16g+2k in the
 *   low nibble and 16g+2k+1 in the high nibble; scale byte g holds S.
 * The RoPE part is copied unchanged.
 *   latent   bf16 [n, 512]        rope      bf16 [n, 64]
 *   dst_row  int64 [n] destination rows, or NULL for rows 0..n-1
 *   kv_codes uint8 [rows, 256]    kv_scales uint8 [rows, 32]
 *   kv_rope  bf16 [rows, 64]
 * n == 0 is a no-op.  Errors: CSA2_ERR_INVALID_ARG for n < 0 or a null
 * pointer (dst_row excepted). */
csa2_status csa2_encode_kv(int64_t n, const uint16_t* latent, const uint16_t* rope,
                           const int64_t* dst_row, uint8_t* kv_codes, uint8_t* kv_scales,
                           uint16_t* kv_rope, void* stream);

/* csa2_encode_kv with `group` (16 or 32) channels per E4M3 scale: the same
 * rule over each group ([akhunji], "Microscopic FP4 (E2M1) Cache
 * Compression", for 32).  kv_scales is uint8 [rows, 512 / group]; codes and
 * rope as in csa2_encode_kv.  Errors: as csa2_encode_kv, and
 * CSA2_ERR_INVALID_ARG for another group. */
csa2_status csa2_encode_kv_grouped(int64_t n, int32_t group, const uint16_t* latent, const uint16_t* rope,
                                   const int64_t* dst_row, uint8_t* kv_codes, uint8_t* kv_scales,
                                   uint16_t* kv_rope, void* stream);

/* FP4 row encode at any width: the per-group codec of csa2_encode_kv applied
 * to rows of `width` channels, without a RoPE part.  It writes the indexer
 * rows of the FP4 indexer calls below ([newsaint] §4: DeepSeek-V4 trained
 * the indexer's query and key with FP4 QAT).
 *   width    16, 32, 64, 128, 256, 512 or 1024
 *   src      bf16 [n, width], 16-byte aligned
 *   dst_row  int64 [n] destination rows, or NULL for rows 0..n-1
 *   codes    uint8 [rows, width / 2], 8-byte aligned
 *   scales   uint8 [rows, width / 16]
 * n == 0 is a no-op.  Errors: CSA2_ERR_INVALID_ARG for n < 0, another width,
 * a null pointer (dst_row excepted) or a misaligned array. */
csa2_status csa2_encode_fp4(int64_t n, int32_t width, const uint16_t* src, const int64_t* dst_row,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* Full-mode indexer, stage 1 of 2: the scan ([atlas] §3.2 hierarchical
 * sparse indexer and mode table; [newsaint] §3: the Full layer scores every
 * causally visible position).  For every query:
 *   s_p = sum_h w_h * max(0, q_h . k_p)  for p in [0, c)   (fp8 inputs on
 *         the fp8 MFMA: the products exact, each 128-long dot product
 *         accumulated inside the instruction, which keeps fewer bits than
 *         fp32 (measured within 3.4e-5 relative of the exact scores on
 *         N(0,1) e4m3 inputs); the weighted sum over heads in fp32)
 *   b_j = max of s_p over p in [8j, min(8j+8, c)),  j < nb = ceil(c / 8)
 *   idx_q        fp8 [n_q, H_i, d_i]      idx_w  float [n_q, H_i]
 *   idx_k        fp8 [rows, d_i]  (one key per position, shared by heads)
 *   block_scores float [n_q, ld_block_scores], 16-byte aligned: b_j
 *                written for j < nb; entries at j >= nb are left untouched;
 *                ld_block_scores >= max(4, ceil((max_visible - W) / 8)) and
 *                a multiple of 4.
 *   pool_ws      optional (NULL, 0): a workspace of
 *                csa2_index_pool_workspace_size bytes.  When given, the scan
 *                also leaves in it what the first pass of csa2_index_pool
 *                computes (each tile's smallest and largest block score, and
 *                a cleared histogram), so that the following csa2_index_pool
 *                call on these block scores, passed the same workspace and
 *                CSA2_POOL_WS_FROM_SCAN, skips that pass; and, per 16 blocks,
 *                the largest block score (as an order key), from which
 *                csa2_pool_topk_attend selects long queries.
 * One kernel.  Queries with n <= W write no block scores. */
csa2_status csa2_index_scan(const csa2_dims* dims, const csa2_queries* q,
                            const uint8_t* idx_q, const float* idx_w, const uint8_t* idx_k,
                            float* block_scores, int64_t ld_block_scores,
                            void* pool_ws, size_t pool_ws_bytes, void* stream);

/* FP4 indexer variant of csa2_index_scan ([newsaint] §4: DeepSeek-V4 trained
 * the indexer's query and key with FP4 QAT).  Same scores and outputs, with
 * the query and key rows in the FP4 format (see the conventions above;
 * csa2_encode_fp4 at width d_i writes them), 72 bytes per key instead of 128:
 *   q_codes  uint8 [n_q, H_i, d_i / 2]   q_scales uint8 [n_q, H_i, d_i / 16]
 *   k_codes  uint8 [rows, d_i / 2]       k_scales uint8 [rows, d_i / 16]
 * Code planes 16-byte aligned, scale planes 8-byte aligned; d_i must be 128
 * (CSA2_ERR_INVALID_ARG otherwise).  Codes times scales are exact in f16 and
 * run the f16 MFMA: the products exact, the sums fp32 (scores within about
 * 2.4e-7 relative of the exact ones). */
csa2_status csa2_index_scan_fp4(const csa2_dims* dims, const csa2_queries* q,
                                const uint8_t* q_codes, const uint8_t* q_scales, const float* idx_w,
                                const uint8_t* k_codes, const uint8_t* k_scales,
                                float* block_scores, int64_t ld_block_scores,
                                void* pool_ws, size_t pool_ws_bytes, void* stream);

/* csa2_index_scan that also keeps every candidate position's score, for a
 * Full layer's own Top-K ([atlas] §3.2 mode table: the Full layer takes a new
 * index set with the query that scored the whole context, so its Top-K in the
 * pool is Reindex with that same query, whose scores the scan has already
 * computed).  FP4 indexer rows when idx_q_scales and idx_k_scales are both
 * given, fp8 when both are NULL; pages NULL for contiguous keys (else as in
 * csa2_index_scan_paged).  Same block scores and pool-workspace preparation
 * as csa2_index_scan, plus:
 *   pos_keys     uint32 [n_q, ld_pos_keys]: position p of query q at
 *                q * ld_pos_keys + p holds the order key of s_p (a uint32
 *                that orders like the score, never 0) for p < c, and 0 for
 *                the positions from c up to c rounded up to 16;
 *                ld_pos_keys a multiple of 32 >= 8 * ceil((max_visible - W)
 *                / 8) rounded up to 32; 16-byte aligned.
 * The scores are bit-identical to csa2_index_reindex's for the same query. */
csa2_status csa2_index_scan_keys(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                 const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                 const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                 float* block_scores, int64_t ld_block_scores,
                                 uint32_t* pos_keys, int64_t ld_pos_keys,
                                 void* pool_ws, size_t pool_ws_bytes, void* stream);

/* A Full layer's Top-K from csa2_index_scan_keys's scores: the same output as
 * csa2_index_reindex called with the scan's indexer query on this pool
 * ([atlas] §3.2), without reading a key.  One kernel, one workgroup per
 * query: the K best pool blocks by (block score desc, block id asc), which
 * hold every one of the K best pool positions (a block ranked above such a
 * position's block brings its own maximum position, ranked above it), then
 * the K best of their positions by (score desc, position asc), ascending.
 *   pool_blocks, pool_count  as written by csa2_index_pool on those scores
 *   block_scores, pos_keys   as written by csa2_index_scan_keys
 *   topk_pos, topk_count, topk_scores  as in csa2_index_reindex. */
csa2_status csa2_index_topk_keys(const csa2_dims* dims, const csa2_queries* q, const int32_t* pool_blocks,
                                 const int32_t* pool_count, const float* block_scores, int64_t ld_block_scores,
                                 const uint32_t* pos_keys, int64_t ld_pos_keys,
                                 int32_t* topk_pos, int32_t* topk_count, float* topk_scores, void* stream);

/* csa2_index_pool followed by csa2_index_topk_keys on its result, in one
 * call: the pool (pool_blocks, pool_count) and the Full layer's Top-K
 * (topk_pos, topk_count) from csa2_index_scan_keys's block scores and
 * position keys, both as those two calls write them.  When every query has
 * at most 16,384 blocks (contexts up to about 131K positions) this is one
 * kernel: the workgroup that selects a query's pool takes its Top-K next,
 * the K best blocks straight from the keys it holds.  Otherwise the chunked
 * pool kernels run, then csa2_index_topk_keys's kernel.
 *   block_scores, pos_keys   as written by csa2_index_scan_keys
 *   ws, flags                as in csa2_index_pool
 * Errors as csa2_index_pool and csa2_index_topk_keys. */
csa2_status csa2_index_pool_topk(const csa2_dims* dims, const csa2_queries* q, const float* block_scores,
                                 int64_t ld_block_scores, const uint32_t* pos_keys, int64_t ld_pos_keys,
                                 int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos,
                                 int32_t* topk_count, void* ws, size_t ws_bytes, int32_t flags, void* stream);

/* csa2_index_pool flag: the workspace was passed to the csa2_index_scan call
 * that wrote these block scores, and since then it was used only by
 * csa2_index_pool calls on the same block scores. */
#define CSA2_POOL_WS_FROM_SCAN 1

/* Workspace bytes for csa2_index_pool (256-byte aligned start required). */
csa2_status csa2_index_pool_workspace_size(const csa2_dims* dims, const csa2_queries* q,
                                           size_t* bytes);

/* Full-mode indexer, stage 2 of 2: the candidate pool ([atlas] §3.2: the
 * Top-2048 blocks of 8 form the pool).  pool = the min(P, nb) blocks with the
 * largest b_j, ties to the lower j, written in ascending block order.
 *   block_scores as written by csa2_index_scan (same alignment and
 *                ld_block_scores rules)
 *   pool_blocks  int32 [n_q, P]  ascending block ids, -1 after pool_count
 *   pool_count   int32 [n_q]     (0 for queries with n <= W)
 *   ws, ws_bytes workspace of csa2_index_pool_workspace_size bytes; its
 *                contents need no initialisation unless flags holds
 *                CSA2_POOL_WS_FROM_SCAN (see csa2_index_scan).
 *   flags        0 or CSA2_POOL_WS_FROM_SCAN.
 * When no query has more than 16,384 blocks: one kernel (one workgroup per
 * query selects from all of its block scores).  Otherwise: a per-chunk key
 * range (skipped with CSA2_POOL_WS_FROM_SCAN), a histogram, and a marking
 * kernel whose last workgroup per query runs the exact final step. */
csa2_status csa2_index_pool(const csa2_dims* dims, const csa2_queries* q,
                            const float* block_scores, int64_t ld_block_scores,
                            int32_t* pool_blocks, int32_t* pool_count,
                            void* ws, size_t ws_bytes, int32_t flags, void* stream);

/* Workspace bytes for csa2_index_full (256-byte aligned start required):
 * the pool workspace followed by room for the block scores. */
csa2_status csa2_index_full_workspace_size(const csa2_dims* dims, const csa2_queries* q,
                                           size_t* bytes);

/* Full-mode indexer: csa2_index_scan followed by csa2_index_pool, the scan
 * preparing the pool workspace (CSA2_POOL_WS_FROM_SCAN).
 *   block_scores  optional float [n_q, ld_block_scores]; NULL keeps the
 *               block scores in the workspace instead.
 *   ws, ws_bytes  workspace of csa2_index_full_workspace_size bytes (when
 *               block_scores is given, csa2_index_pool_workspace_size bytes
 *               suffice). */
csa2_status csa2_index_full(const csa2_dims* dims, const csa2_queries* q,
                            const uint8_t* idx_q, const float* idx_w, const uint8_t* idx_k,
                            int32_t* pool_blocks, int32_t* pool_count,
                            float* block_scores, int64_t ld_block_scores,
                            void* ws, size_t ws_bytes, void* stream);

/* csa2_index_full with FP4 indexer rows (as csa2_index_scan_fp4); the same
 * workspace size. */
csa2_status csa2_index_full_fp4(const csa2_dims* dims, const csa2_queries* q,
                                const uint8_t* q_codes, const uint8_t* q_scales, const float* idx_w,
                                const uint8_t* k_codes, const uint8_t* k_scales,
                                int32_t* pool_blocks, int32_t* pool_count,
                                float* block_scores, int64_t ld_block_scores,
                                void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for csa2_index_reindex. */
csa2_status csa2_index_reindex_workspace_size(const csa2_dims* dims, const csa2_queries* q,
                                              size_t* bytes);

/* Reindex inside the pool ([atlas] §3.2: Reindex re-scores with this
 * layer's indexer query over the pool only and keeps the Top-K; [newsaint]
 * §3 constant-size search domain; §8 gathers only the pool's keys).
 * Candidates R = union over pool blocks j of [8j, min(8j+8, c)); scores as
 * in csa2_index_full with this call's (idx_q, idx_w); keeps the
 * min(K, |R|) best by (score desc, position asc), ascending positions.
 *   pool_blocks, pool_count  as produced by csa2_index_full (ascending)
 *   topk_pos    int32 [n_q, K]  ascending positions, -1 after topk_count
 *   topk_count  int32 [n_q]
 *   topk_scores optional float [n_q, K] (NULL to skip): the score of each
 *               kept position, same order as topk_pos.
 *   ws, ws_bytes  workspace of csa2_index_reindex_workspace_size bytes.  Its
 *               first bytes are per-query completion counters of the
 *               scoring workgroups: they must be zero before the first call
 *               on a workspace (allocate it zero-filled), and every call
 *               leaves them zero.  Calls sharing a workspace must be ordered
 *               on one stream.
 * One kernel: the last scoring workgroup of each query selects its Top-K. */
csa2_status csa2_index_reindex(const csa2_dims* dims, const csa2_queries* q,
                               const uint8_t* idx_q, const float* idx_w, const uint8_t* idx_k,
                               const int32_t* pool_blocks, const int32_t* pool_count,
                               int32_t* topk_pos, int32_t* topk_count, float* topk_scores,
                               void* ws, size_t ws_bytes, void* stream);

/* csa2_index_reindex with FP4 indexer rows (as csa2_index_scan_fp4); the
 * same workspace size and contract. */
csa2_status csa2_index_reindex_fp4(const csa2_dims* dims, const csa2_queries* q,
                                   const uint8_t* q_codes, const uint8_t* q_scales, const float* idx_w,
                                   const uint8_t* k_codes, const uint8_t* k_scales,
                                   const int32_t* pool_blocks, const int32_t* pool_count,
                                   int32_t* topk_pos, int32_t* topk_count, float* topk_scores,
                                   void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for csa2_attend: 0 when each (query, 32-head group) is one
 * workgroup, else the partials of its splits (2 KiB + 8 B per split and
 * head, heads padded to a multiple of 32).  The split count depends only on
 * n_q, n_heads, topk and swa: one split per 64-entry tile for a batch of a
 * few queries, one per (query, head group) once n_q * ceil(H / 32) >= 256. */
csa2_status csa2_attend_workspace_size(const csa2_dims* dims, const csa2_queries* q,
                                       size_t* bytes);

/* Core attention, MLA-absorbed, over the kept FP4 entries and the window
 * ([atlas] §3.2 heterogeneous KV: one main Q attends the sparse main-KV
 * branch and the uncompressed window branch, merged; mode table: Reuse
 * layers call this with a new Q and the inherited index set; [newsaint] §4:
 * FP4 is dequantised just before attention).  Entries of a query:
 *   sparse  j in topk_pos[0 .. topk_count): key = [deq(codes, scales) (512)
 *           || kv_rope (64)], value = deq latent (512);
 *   window  positions [c, n) read from swa_kv rows swa_base .. swa_base+n-c-1:
 *           key = the row's 576 bf16 values, value = its first 512.
 *   l_j = softmax_scale * (q_lat . key[:512] + q_rope . key[512:]);
 *   out_h = sum_j softmax(l)_j value_j  (one softmax over all entries),
 *   lse_h = log sum_j exp(l_j).  A query with no entries gets out = 0 and
 *   lse = -inf.
 *   q_lat  bf16 [n_q, H, 512]     q_rope bf16 [n_q, H, 64]
 *   kv_codes, kv_scales, kv_rope  as written by csa2_encode_kv (kv_scales
 *          [rows, 512 / kv_group]; csa2_encode_kv_grouped for kv_group 32)
 *   topk_pos, topk_count          as produced by csa2_index_reindex
 *   swa_kv bf16 [swa_rows, 576]   swa_base int64 [n_q] (device)
 *   out    float [n_q, H, 512]    lse float [n_q, H] or NULL
 *   ws, ws_bytes  csa2_attend_workspace_size bytes (NULL when that is 0),
 *          256-byte aligned, no initial contents; calls sharing it must be
 *          ordered on one stream.
 * One kernel, or two when the plan splits a query's entries (the second
 * merges the splits with a log-sum-exp rescale).
 * Window values are converted to fp16 for the value product: |v| must stay
 * below 65504. */
csa2_status csa2_attend(const csa2_dims* dims, const csa2_queries* q,
                        const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                        const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                        const int32_t* topk_pos, const int32_t* topk_count,
                        const uint16_t* swa_kv, const int64_t* swa_base,
                        float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* csa2_index_reindex over paged indexer keys (see csa2_pages): the same
 * selection from the same scores.  FP4 indexer rows when idx_q_scales and
 * idx_k_scales are both given (as csa2_index_reindex_fp4), fp8 when both are
 * NULL.  Same workspace as csa2_index_reindex.  One extra dependent load per
 * pool position (its page id) before the key gather. */
csa2_status csa2_index_reindex_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                     const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                     const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                     const int32_t* pool_blocks, const int32_t* pool_count,
                                     int32_t* topk_pos, int32_t* topk_count, float* topk_scores,
                                     void* ws, size_t ws_bytes, void* stream);

/* csa2_index_scan over paged indexer keys (see csa2_pages): the same block
 * scores, and the same pool-workspace preparation when pool_ws is given.
 * FP4 rows when idx_q_scales and idx_k_scales are both given, fp8 when both
 * are NULL. */
csa2_status csa2_index_scan_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                  const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                  const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                  float* block_scores, int64_t ld_block_scores,
                                  void* pool_ws, size_t pool_ws_bytes, void* stream);

/* csa2_index_full over paged indexer keys (see csa2_pages): the same block
 * scores and pool.  Each scan workgroup first loads its tile's page ids (one
 * extra round trip before its key stream starts); every 16-position step of
 * the stream then reads 16 rows of one page.  FP4 rows when idx_q_scales and
 * idx_k_scales are both given, fp8 when both are NULL.  Same workspace as
 * csa2_index_full. */
csa2_status csa2_index_full_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                  const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                  const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                  int32_t* pool_blocks, int32_t* pool_count,
                                  float* block_scores, int64_t ld_block_scores,
                                  void* ws, size_t ws_bytes, void* stream);

/* csa2_attend over paged main-KV planes (see csa2_pages): the same outputs
 * from the same entries; the kept positions are turned into rows (one page
 * id load each) before the FP4 gather.  The window rows come from swa_kv at
 * swa_base as in csa2_attend.  Same workspace as csa2_attend. */
csa2_status csa2_attend_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                              const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                              const int32_t* topk_pos, const int32_t* topk_count,
                              const uint16_t* swa_kv, const int64_t* swa_base,
                              float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* csa2_index_pool_topk followed by csa2_attend on its Top-K, with the Top-K
 * selected inside the attention kernel: every attention workgroup that
 * holds kept-entry tiles selects its query's Top-K itself from the scan's
 * scores and gathers its tiles' entries at once, so no launch and no round
 * trip for the positions sit between the selection and the gathers.  When
 * every query has at most 16,384 blocks (contexts up to about 131K
 * positions) the pool is selected there too (the same selection as
 * csa2_index_pool_topk's one-workgroup kernel, repeated by each such
 * workgroup): one attention launch for the whole chain.  Longer queries
 * (up to 131,072 blocks, contexts up to about 1M positions) after a scan
 * that prepared pool_ws (flags CSA2_POOL_WS_FROM_SCAN) are selected in the
 * same launch from the scan's group keys (the largest block score of every
 * 16 blocks, which pool_ws holds): one extra workgroup per query writes the
 * pool, and the attention workgroups take the Top-K's candidates from the
 * groups at or above a bound of the K-th group key; the result is exact
 * (candidates that overflow their room fall back to an exact selection that
 * streams every block score).  Otherwise the chunked pool kernels run first
 * and the attention workgroups select the Top-K of that pool (as
 * csa2_index_topk_keys).  pool_blocks and pool_count are written as
 * csa2_index_pool_topk writes them, and the workgroup holding head group 0's
 * first kept-entry tile writes topk_pos and topk_count; out and lse are
 * csa2_attend's on that Top-K.
 *   block_scores, pos_keys   as written by csa2_index_scan_keys
 *   q_lat ... lse            as in csa2_attend (topk_pos, topk_count are
 *                            outputs here)
 *   pool_ws, pool_ws_bytes, flags  as ws, ws_bytes, flags of
 *                            csa2_index_pool (read only for queries past
 *                            16,384 blocks; NULL and 0 are accepted for
 *                            small pools)
 *   ws, ws_bytes             csa2_attend_workspace_size bytes, as in csa2_attend
 * Errors as csa2_index_pool_topk and csa2_attend. */
csa2_status csa2_pool_topk_attend(const csa2_dims* dims, const csa2_queries* q, const float* block_scores,
                                  int64_t ld_block_scores, const uint32_t* pos_keys, int64_t ld_pos_keys,
                                  int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                  const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                                  const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                                  const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                                  void* pool_ws, size_t pool_ws_bytes, int32_t flags,
                                  void* ws, size_t ws_bytes, void* stream);

/* csa2_pool_topk_attend over paged main-KV planes (see csa2_pages; NEXT-3
 * paged caches): the same selection from the same block scores and position
 * keys (as csa2_index_scan_keys writes them with pages), after which each
 * selecting workgroup turns its kept positions into rows of the planes with
 * one page-id load each before its gathers; pool_blocks, pool_count,
 * topk_pos and topk_count hold positions, as in the unpaged call.  Same
 * arguments otherwise; errors as csa2_attend_paged for the pages. */
csa2_status csa2_pool_topk_attend_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                        const float* block_scores, int64_t ld_block_scores, const uint32_t* pos_keys,
                                        int64_t ld_pos_keys, int32_t* pool_blocks, int32_t* pool_count,
                                        int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat,
                                        const uint16_t* q_rope, float softmax_scale, const uint8_t* kv_codes,
                                        const uint8_t* kv_scales, const uint16_t* kv_rope, const uint16_t* swa_kv,
                                        const int64_t* swa_base, float* out, float* lse, void* pool_ws,
                                        size_t pool_ws_bytes, int32_t flags, void* ws, size_t ws_bytes,
                                        void* stream);

/* csa2_index_reindex followed by csa2_attend on its Top-K, with the Top-K
 * selected inside the attention kernel: the Reindex kernel only scores the
 * pool's positions (order keys into reindex_ws), and every attention
 * workgroup that holds kept-entry tiles selects the K best of them itself
 * (the same selection as csa2_index_reindex's) and gathers its tiles'
 * entries at once.  The workgroup holding head group 0's first kept-entry
 * tile writes topk_pos and topk_count, as csa2_index_reindex writes them
 * ([atlas] §3.2: a Reindex layer re-scores the inherited pool with its own
 * indexer query, then attends over the kept positions with its main Q).
 * FP4 indexer rows when idx_q_scales and idx_k_scales are both given.
 *   idx_q ... pool_count          as in csa2_index_reindex
 *   q_lat ... lse                 as in csa2_attend (topk_pos, topk_count
 *                                 are outputs here)
 *   reindex_ws, reindex_ws_bytes  csa2_index_reindex_workspace_size bytes
 *                                 (its completion counters are not used)
 *   ws, ws_bytes                  csa2_attend_workspace_size bytes
 * Errors as those two calls. */
csa2_status csa2_reindex_attend(const csa2_dims* dims, const csa2_queries* q, const uint8_t* idx_q,
                                const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                                const uint8_t* idx_k_scales, const int32_t* pool_blocks, const int32_t* pool_count,
                                int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                                float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base,
                                float* out, float* lse, void* reindex_ws, size_t reindex_ws_bytes,
                                void* ws, size_t ws_bytes, void* stream);

/* csa2_reindex_attend over paged planes (see csa2_pages): the Reindex
 * scoring reads the pool's keys through the page table (as
 * csa2_index_reindex_paged) and each selecting attention workgroup turns its
 * kept positions into rows with one page-id load each before its gathers.
 * Same arguments and outputs (positions) otherwise. */
csa2_status csa2_reindex_attend_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                      const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                      const uint8_t* idx_k, const uint8_t* idx_k_scales, const int32_t* pool_blocks,
                                      const int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                      const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                                      const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                                      const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                                      void* reindex_ws, size_t reindex_ws_bytes, void* ws, size_t ws_bytes,
                                      void* stream);

/* Rows of paged positions, so that csa2_encode_kv (through dst_row) appends
 * new entries into their pages:
 *   dst_row[i] = table[table_off[i] + pos[i] / page_size] * page_size
 *                + pos[i] % page_size
 *   table_off  device int64 [n]   pos  device int32 [n] (>= 0)
 *   dst_row    device int64 [n]   (output)
 * One kernel. */
csa2_status csa2_page_rows(const csa2_pages* pages, int64_t n, const int64_t* table_off, const int32_t* pos,
                           int64_t* dst_row, void* stream);

/* One decode layer in one call ([atlas] §3.2 mode table: a Full layer
 * scores the whole context and takes a new index set, a Reindex layer
 * re-scores the inherited pool with its own indexer query, a Reuse layer
 * only attends over the inherited index set with its own main Q).  The call
 * checks every stage's arguments, then enqueues, on `stream`:
 *   CSA2_LAYER_FULL     csa2_index_scan_keys, then csa2_pool_topk_attend
 *                       (pool_blocks, pool_count, and topk_pos,
 *                       topk_count: the same set as csa2_index_reindex
 *                       with the same indexer query);
 *   CSA2_LAYER_REINDEX  csa2_reindex_attend on the given pool;
 *   CSA2_LAYER_REUSE    csa2_attend on the given topk_pos / topk_count
 *                       (the idx_* arguments may be NULL).
 * The indexer rows are fp8 when idx_q_scales and idx_k_scales are NULL and
 * FP4 (as the *_fp4 calls) when both are given.  Every other argument is as
 * in the stage calls.  The chain is the stages' own launches, which a caller
 * can also capture into a HIP graph (no memset or allocation is enqueued).
 *   ws, ws_bytes  csa2_decode_step_workspace_size bytes, 256-byte aligned,
 *               zero-filled before its first use (it holds the Reindex
 *               completion counters, which every call leaves at zero);
 *               calls sharing it must be ordered on one stream. */
#define CSA2_LAYER_FULL 0
#define CSA2_LAYER_REINDEX 1
#define CSA2_LAYER_REUSE 2

csa2_status csa2_decode_step_workspace_size(const csa2_dims* dims, const csa2_queries* q, size_t* bytes);

/* csa2_decode_step with every per-position plane paged (see csa2_pages):
 * the stages' paged calls (csa2_index_scan_keys with pages,
 * csa2_pool_topk_attend_paged, csa2_reindex_attend_paged, csa2_attend_paged)
 * in the same order and with the same workspace. */
csa2_status csa2_decode_step_paged(const csa2_dims* dims, const csa2_queries* q, const csa2_pages* pages,
                                   int32_t mode, const uint8_t* idx_q, const uint8_t* idx_q_scales,
                                   const float* idx_w, const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                   int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos,
                                   int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                                   float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                   const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base,
                                   float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

csa2_status csa2_decode_step(const csa2_dims* dims, const csa2_queries* q, int32_t mode,
                             const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                             const uint8_t* idx_k, const uint8_t* idx_k_scales,
                             int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                             const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                             const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                             const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* csa2_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid allocation.  The same stages, kernels and outputs
 * as csa2_decode_step; the scratch they need (pool workspace, block scores,
 * Reindex order keys and completion counters, attention partials) comes from
 * one array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends.  The call allocates nothing.
 *   Limits: at most 65,536 queries, and a batch whose workspace
 *   (csa2_decode_step_workspace_size) fits in 64 MiB minus 256 KiB: batch 1
 *   at 1M context takes about 6 MiB, batch 8 at 128K about 16 MiB, 32
 *   queries of up to 256K about 56 MiB.  Larger batches get
 *   CSA2_ERR_WORKSPACE, enqueuing
 *   nothing.
 *   Every call on one GPU uses that GPU's array: calls that may overlap on
 *   one GPU (different streams, or a graph replayed while another call runs)
 *   race and must be ordered by the caller.  Other errors as
 *   csa2_decode_step. */
csa2_status csa2_decode_step_noalloc(const csa2_dims* dims, const csa2_queries* q, int32_t mode,
                                     const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                     const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                     int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos,
                                     int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                                     float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                     const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base,
                                     float* out, float* lse, void* stream);

/* Measurement helper, not a step of the method: reads `bytes` bytes of
 * device memory at `buf` once (16-byte nontemporal loads into registers, two
 * workgroups per CU, each over one contiguous chunk) and writes nothing,
 * except that `sink` (a device word) may receive a value in a case that
 * does not arise for any data.  Timing it gives the streaming-read rate of
 * this GPU's HBM that the Full scan's bandwidth is compared with.
 *   buf    16-byte aligned; bytes a multiple of 16 (0 is a no-op)
 *   sink   4-byte aligned device word
 * Errors: CSA2_ERR_INVALID_ARG for a bad size, NULL or misaligned pointer. */
csa2_status csa2_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
