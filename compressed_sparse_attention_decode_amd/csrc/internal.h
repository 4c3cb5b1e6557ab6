// Launchers shared between the host dispatch and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "scan_args.h"

namespace csa2 {

struct PoolArgs {
  const float* bscore;
  int64_t ld;
  const int32_t* n_visible;
  int n_q, swa, pool;
  int chunks;                // kPoolChunk-block chunks per query (grid of K1, K2)
  int mark_wgs;              // marking workgroups per query (1..chunks; each takes a run of chunks)
  uint32_t* ws;              // [n_q, ws_stride] words (histogram, chunk results)
  int64_t ws_stride;
  int mm_cap;                // (min, max) key pairs per query in the workspace
  int mm_half;               // pairs [0, mm_half) cover mm_span1 blocks each, later pairs mm_span
  int mm_span1;
  int mm_span;               // blocks covered by one pair (after the first mm_half)
  bool have_minmax;          // pairs and a cleared histogram already written (by the scan)
  int nw_cap;                // bitmap words of the longest query's blocks (final step LDS)
  bool small;                // every query has <= kPoolSmallBlocks blocks: one-workgroup selection
  int32_t* pool_blocks;      // [n_q, pool]
  int32_t* pool_count;
  // optional (topk_pos != nullptr, small pools only): the Full layer's
  // Top-K from the scan's position keys, in the selecting workgroup
  const uint32_t* pkey;      // [n_q, ld_pkey]
  int64_t ld_pkey;
  int topk;
  int32_t* topk_pos;         // [n_q, topk]
  int32_t* topk_count;
};

struct ReindexArgs {
  const uint8_t* idx_q;      // fp8 [n_q, Hi, d], or FP4 codes [n_q, Hi, d / 2]
  const float* idx_w;
  const uint8_t* idx_k;      // fp8 [rows, d], or FP4 codes [rows, d / 2]
  const uint8_t* idx_q_scales;   // FP4 rows (nullptr: fp8): [n_q, Hi, d / 16]
  const uint8_t* idx_k_scales;   // [rows, d / 16]
  const int64_t* seq_base;
  const int32_t* n_visible;
  const int32_t* pool_blocks;
  const int32_t* pool_count;
  int n_q, hi, d, swa, pool, topk;
  int split;                 // scoring workgroups per query
  int blocks_per_wg;         // pool blocks per scoring workgroup (kReindexBlocks or kReindexBlocksWide)
  uint32_t* done;            // workspace [n_q]: scoring workgroups finished (zero between calls)
  uint32_t* keys;            // workspace [n_q, 8 * pool]: order keys, 0 = empty
  int32_t* topk_pos;
  int32_t* topk_count;
  float* topk_scores;        // optional
  int score_only;            // 1: only the keys (the attention kernel selects from them)
  // paged caches (nullptr: position p of query q's sequence is row
  // seq_base[q] + p): it is row (pages[seq_base[q] + (p >> page_shift)] <<
  // page_shift) + (p mod 2^page_shift) of planes of `rows` rows
  const int32_t* pages;
  int page_shift;
  int64_t rows;
};

struct AttendArgs {
  const uint16_t* q_lat;     // [n_q, H, 512]
  const uint16_t* q_rope;    // [n_q, H, 64]
  float scale_log2;          // softmax_scale * log2(e)
  const uint8_t* kv_codes;
  const uint8_t* kv_scales;  // [rows, 512 >> (4 + kv_gshift)]
  int kv_gshift;             // FP4 scale group: 16 << kv_gshift channels (0 or 1)
  const uint16_t* kv_rope;
  const int32_t* topk_pos;
  const int32_t* topk_count;
  const uint16_t* swa_kv;
  const int64_t* swa_base;
  const int64_t* seq_base;
  const int32_t* n_visible;
  int n_q, heads, topk, swa;
  int head_groups;           // workgroups across heads per query (32 heads each)
  int splits;                // workgroups across the tile list per query and head group
  int split_tiles;           // tiles per split (the window's tiles first, then the kept entries')
  float* out;                // [n_q, H, 512]
  float* lse;                // optional [n_q, H]
  float* part_o;             // splits > 1: [n_q][splits][head_groups * 32][512] unnormalised o
  float* part_ml;            // splits > 1: [n_q][splits][head_groups * 32][2] (m in the exp2 domain, l)
  const int32_t* pages;      // paged main-KV planes (as ReindexArgs; the window stays apart)
  int page_shift;
  int64_t rows;
  // the pool and the Full layer's Top-K selected in the attention kernel
  // (bscore != nullptr; then topk_pos / topk_count are not read): the scan's
  // block scores and position keys, and where the selection goes
  const float* bscore;
  int64_t ld_bs;
  const uint32_t* pkey;
  int64_t ld_pkey;
  int pool;
  int32_t* pool_blocks;
  int32_t* pool_count;
  int32_t* topk_out;         // [n_q, topk]
  int32_t* topk_count_out;
  int sel_from_pool;         // 1: the pool is given (pool_blocks, pool_count are read), only the Top-K is selected
  const uint32_t* rkeys;     // Reindex order keys [n_q, 8 * pool] (csa2_reindex_attend): the Top-K from them
  // the scan's group keys (nullptr: none): a query of more than kMaxCand
  // blocks selects from them, query q's at gkey + q * ld_gkey, gcap words
  const uint32_t* gkey;
  int64_t ld_gkey;
  int gcap;
  int group_min;             // queries of more blocks take the Top-K from the group keys (<= kMaxCand)
};

// A Full layer's Top-K from the Full scan's own scores (the same indexer
// query as the scan, so the same scores Reindex would compute).
struct TopkKeysArgs {
  const int32_t* pool_blocks;   // [n_q, pool] ascending, -1 past the count
  const int32_t* pool_count;
  const float* bscore;          // [n_q, ld] block scores written by the scan
  int64_t ld;
  const uint32_t* pkey;         // [n_q, ld_pkey] position keys written by the scan
  int64_t ld_pkey;
  int n_q, pool, topk;
  int32_t* topk_pos;
  int32_t* topk_count;
  float* topk_scores;           // optional
};

hipError_t launch_encode(int64_t n, int group, const uint16_t* latent, const uint16_t* rope,
                         const int64_t* dst_row, uint8_t* codes, uint8_t* scales,
                         uint16_t* rope_out, hipStream_t s);
hipError_t launch_encode_rows(int64_t n, int width, const uint16_t* src, const int64_t* dst_row,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_page_rows(int64_t n, const int32_t* pages, int page_shift, const int64_t* table_off,
                            const int32_t* pos, int64_t* dst_row, hipStream_t s);
hipError_t launch_pool_select(const PoolArgs& a, hipStream_t s);
int64_t pool_ws_words(int chunks, int mm_cap);   // workspace words per query
int64_t pool_gkey_off(int chunks, int mm_cap);   // word offset of the group keys in a query's workspace
hipError_t launch_reindex(const ReindexArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
hipError_t launch_topk_keys(const TopkKeysArgs& a, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t s);

// Tiling constants the host needs for grids and workspace sizes.
constexpr int kPoolChunk = 4096;       // blocks per pool-select chunk workgroup
constexpr int kPoolChunkCand = 1024;   // candidate slots per chunk
constexpr int kPoolSmallBlocks = 16384;   // blocks a one-workgroup pool selection holds
constexpr int kPoolGroupsMax = 8192;      // group keys an in-kernel selection holds (131,072 blocks)
constexpr int kAttendTile = 64;        // entries per attention tile
constexpr int kAttendWaves = 8;        // waves per attention workgroup (two groups of 16 heads, 4 waves each)
constexpr int kAttendHeads = 32;       // heads per attention workgroup
constexpr int kAttendMaxSplits = 16;   // tile-list splits per query and head group, at most
constexpr int kAttendMaxTiles = 48;    // tiles of one query: 1024 / 64 window + 2048 / 64 kept
constexpr int kReindexBlocks = 64;     // pool blocks per Reindex scoring workgroup (one-round grids)
constexpr int kReindexBlocksWide = 128;   // ... when 64-block workgroups would exceed two per CU
constexpr int kReindexBlocksNarrow = 32;  // ... when 32-block workgroups fit in one per CU
constexpr int kReindexBlocksHuge = 256;   // ... when 128-block workgroups would exceed one per CU
constexpr int kMaxVisible = 1 << 21;   // bound of n_visible
constexpr int kMaxTokensPerSeq = 64;   // query tokens of one sequence sharing its key stream
constexpr int kMaxBlocks = kMaxVisible / 8;

}  // namespace csa2
