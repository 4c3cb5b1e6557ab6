// C ABI of the CSA2 decode-path library: argument checks, workspace layout and
// kernel launches.  Declarations and contracts are in include/csa2.h.
#include <algorithm>
#include <mutex>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/csa2.h"
#include "internal.h"

using namespace csa2;

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa2_status hip_fail(hipError_t e, const char* what) {
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Per-device properties, filled once under check_device's lock (before the
// device is marked known) and read only after a successful check_device.
int g_cus[64] = {0};                 // compute units per checked device

// gfx950 check, once per device.
csa2_status check_device() {
  static std::mutex mu;
  static int known[64] = {0};        // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(CSA2_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    known[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev] = p.multiProcessorCount;
  }
  if (known[dev] != 1) return fail(CSA2_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return CSA2_OK;
}

csa2_status check_dims(const csa2_dims* d) {
  if (!d) return fail(CSA2_ERR_INVALID_ARG, "dims is NULL");
  if (d->d_latent != 512) return fail(CSA2_ERR_INVALID_ARG, "d_latent must be 512 (got %d)", d->d_latent);
  if (d->d_rope != 64) return fail(CSA2_ERR_INVALID_ARG, "d_rope must be 64 (got %d)", d->d_rope);
  if (d->block != 8) return fail(CSA2_ERR_INVALID_ARG, "block must be 8 (got %d)", d->block);
  if (d->n_heads < 8 || d->n_heads > 128 || d->n_heads % 8)
    return fail(CSA2_ERR_INVALID_ARG, "n_heads must be a multiple of 8 in [8, 128] (got %d)", d->n_heads);
  if (d->idx_heads < 1 || d->idx_heads > 64)
    return fail(CSA2_ERR_INVALID_ARG, "idx_heads must be in [1, 64] (got %d)", d->idx_heads);
  if (d->idx_dim != 64 && d->idx_dim != 128)
    return fail(CSA2_ERR_INVALID_ARG, "idx_dim must be 64 or 128 (got %d)", d->idx_dim);
  if (d->pool_blocks < 1 || d->pool_blocks > 2048)
    return fail(CSA2_ERR_INVALID_ARG, "pool_blocks must be in [1, 2048] (got %d)", d->pool_blocks);
  if (d->topk < 1 || d->topk > 2048 || d->topk > 8 * d->pool_blocks)
    return fail(CSA2_ERR_INVALID_ARG, "topk must be in [1, min(2048, 8*pool_blocks)] (got %d)", d->topk);
  if (d->swa < 0 || d->swa > 1024) return fail(CSA2_ERR_INVALID_ARG, "swa must be in [0, 1024] (got %d)", d->swa);
  if (d->kv_group != 0 && d->kv_group != 16 && d->kv_group != 32)
    return fail(CSA2_ERR_INVALID_ARG, "kv_group must be 0, 16 or 32 (got %d)", d->kv_group);
  return CSA2_OK;
}

csa2_status check_queries(const csa2_queries* q) {
  if (!q) return fail(CSA2_ERR_INVALID_ARG, "queries is NULL");
  if (q->n_q < 1) return fail(CSA2_ERR_INVALID_ARG, "n_q must be >= 1 (got %d)", q->n_q);
  if (q->n_q > (1 << 20)) return fail(CSA2_ERR_INVALID_ARG, "n_q must be <= 2^20 (got %d)", q->n_q);
  if (q->tokens_per_seq < 1 || q->tokens_per_seq > kMaxTokensPerSeq || q->n_q % q->tokens_per_seq)
    return fail(CSA2_ERR_INVALID_ARG, "tokens_per_seq must be 1..%d and divide n_q (got %d)", kMaxTokensPerSeq,
                q->tokens_per_seq);
  if (q->max_visible < 0 || q->max_visible > kMaxVisible)
    return fail(CSA2_ERR_INVALID_ARG, "max_visible must be in [0, 2^21] (got %d)", q->max_visible);
  if (q->reserved != 0) return fail(CSA2_ERR_INVALID_ARG, "reserved must be 0");
  if (!q->seq_base || !q->n_visible) return fail(CSA2_ERR_INVALID_ARG, "seq_base / n_visible is NULL");
  return CSA2_OK;
}

// Paged planes: the page table, a power-of-two page, and planes whose byte
// offsets (rows x the widest plane's row bytes) stay inside one 32-bit
// buffer range, as the gathers address them.
csa2_status check_pages(const csa2_pages* p, int64_t row_bytes) {
  if (!p || !p->table) return fail(CSA2_ERR_INVALID_ARG, "pages / pages->table is NULL");
  if (p->reserved != 0) return fail(CSA2_ERR_INVALID_ARG, "pages->reserved must be 0");
  if (p->page_size < 16 || p->page_size > 65536 || (p->page_size & (p->page_size - 1)))
    return fail(CSA2_ERR_INVALID_ARG, "page_size must be a power of two in [16, 65536] (got %d)", p->page_size);
  if (p->rows < 1 || p->rows % p->page_size)
    return fail(CSA2_ERR_INVALID_ARG, "pages->rows must be a positive multiple of page_size (got %lld)",
                (long long)p->rows);
  if (p->rows > (int64_t)0xFFFFFF00 / row_bytes)
    return fail(CSA2_ERR_INVALID_ARG, "paged planes of %lld rows x %lld bytes exceed the 4 GiB gather range",
                (long long)p->rows, (long long)row_bytes);
  return CSA2_OK;
}

int page_shift(const csa2_pages* p) { return __builtin_ctz((unsigned)p->page_size); }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t max_blocks(const csa2_dims* d, const csa2_queries* q) {
  const int64_t c = q->max_visible > d->swa ? q->max_visible - d->swa : 0;
  return (c + 7) / 8;
}

// index_full workspace: block scores n_q x ldb f32 (when the caller passes none)
int64_t full_ldb(const csa2_dims* d, const csa2_queries* q) {
  const int64_t nb = max_blocks(d, q);
  return ((nb > 0 ? nb : 1) + 63) / 64 * 64;
}

int pool_chunks(const csa2_dims* d, const csa2_queries* q) {
  const int64_t nb = max_blocks(d, q);
  const int64_t g = (nb + kPoolChunk - 1) / kPoolChunk;
  return g > 0 ? (int)g : 1;
}

// Positions per Full-scan workgroup: kScanTile, halved (down to 128) while
// the launch would hold fewer than kScanSmallGrid workgroups, so that a few
// short queries spread over more CUs instead of each wave walking a long run
// of positions alone.  A function of the sizes only, so the scan, the pool
// that reads its key ranges and the workspace sizes agree
// (CSA2_SCAN_TILE overrides for tuning).
int scan_tile(const csa2_dims* d, const csa2_queries* q) {
  int tile = kScanTile;
  const int64_t pos = max_blocks(d, q) * 8;
  while (tile > kScanTileMin && (int64_t)q->n_q * ((pos + tile - 1) / tile) < kScanSmallGrid) tile /= 2;
  if (const char* env = getenv("CSA2_SCAN_TILE")) tile = atoi(env);
  if (tile < 64 || tile % 64 || tile > 4096) tile = kScanTile;
  return tile;
}

int scan_tiles(const csa2_dims* d, const csa2_queries* q, int tile) {
  return (int)((max_blocks(d, q) * 8 + tile - 1) / tile);
}

// Uneven scan tiles: when the whole grid is one round of at most two
// workgroups per CU, the first-dispatched workgroup on a CU streams faster
// than the second, so the first half of the tiles take kScanTileExtra more
// positions and the second half as many fewer (measured: 0.4 us at 8 x 128K,
// 1 us at 1M).  CSA2_SCAN_SPLIT overrides the shift (0 disables it).  Called
// after check_device; the scan and the pool that reads its key ranges agree.
int scan_tile_extra(const csa2_dims* d, const csa2_queries* q, int tile, int tiles) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int64_t units = ((int64_t)(q->n_q / q->tokens_per_seq) * tiles + 7) / 8 * 8;
  int extra = units * q->tokens_per_seq <= 2 * (int64_t)g_cus[dev] ? kScanTileExtra : 0;
  if (const char* env = getenv("CSA2_SCAN_SPLIT")) extra = atoi(env);
  if (extra < 0 || extra % 16 || extra >= tile || tile + extra > 4096 || (tiles & 1)) extra = 0;
  return extra;
}

// (min, max) key pairs per query: one per pool chunk or one per scan tile
int pool_mm_cap(const csa2_dims* d, const csa2_queries* q) {
  const int t = scan_tiles(d, q, scan_tile(d, q)), g = pool_chunks(d, q);
  return t > g ? t : g;
}

// The scan writes group keys (the largest block key of each kGroupBlocks
// blocks) into the pool workspace when its tiles start at group boundaries:
// always, unless CSA2_SCAN_TILE / CSA2_SCAN_SPLIT move them off.
static bool scan_groups_ok(const csa2_dims* d, const csa2_queries* q) {
  const int tile = scan_tile(d, q), tiles = scan_tiles(d, q, tile);
  const int extra = scan_tile_extra(d, q, tile, tiles);
  return tile % (8 * kGroupBlocks) == 0 && extra % (8 * kGroupBlocks) == 0;
}

// Words of a query's group keys in the pool workspace.
static int pool_gcap(const csa2_dims* d, const csa2_queries* q) { return pool_chunks(d, q) * (kPoolChunk / kGroupBlocks); }

size_t pool_ws(const csa2_dims* d, const csa2_queries* q) {
  return align256((size_t)q->n_q * pool_ws_words(pool_chunks(d, q), pool_mm_cap(d, q)) * 4);
}

// index_full workspace: the pool workspace, then block scores n_q x ldb f32
// (used when the caller passes none)
size_t full_ws(const csa2_dims* d, const csa2_queries* q) {
  return pool_ws(d, q) + align256((size_t)q->n_q * full_ldb(d, q) * 4);
}

// A Full layer's position keys (decode step): n_q x (8 x the block-score
// stride) order keys, one per candidate position
int64_t full_ldpk(const csa2_dims* d, const csa2_queries* q) { return full_ldb(d, q) * 8; }
size_t pkey_ws(const csa2_dims* d, const csa2_queries* q) {
  return align256((size_t)q->n_q * full_ldpk(d, q) * 4);
}

// Reindex workspace: per-query completion counters (zero between calls),
// then the order keys n_q x 8P u32
size_t reindex_keys_ws(const csa2_dims* d, const csa2_queries* q) {
  return align256((size_t)q->n_q * d->pool_blocks * 8 * 4);
}
size_t reindex_ws(const csa2_dims* d, const csa2_queries* q) {
  return align256((size_t)q->n_q * 4) + reindex_keys_ws(d, q);
}

// Pool blocks per Reindex scoring workgroup: 32 when 32-block workgroups
// fit in one per CU (a batch of a few queries: more of them share the
// scoring), 64 when 64-block workgroups fit in two per CU, 128 when 128-block
// ones fit in one per CU (their registers allow one), else 256 (one round of
// one workgroup per CU, where 128-block ones would take two).
// Measured per Reindex call: 1 query 14.4 / 15.4 us (32 / 64), 8 queries
// 19.2 / 25.8 us (64 / 32), 32 queries 42.5 / 56.9 us (128 / 64).
// CSA2_REINDEX_BLOCKS (32, 64, 128 or 256) overrides.  Called after
// check_device.
int reindex_blocks_per_wg(const csa2_dims* d, const csa2_queries* q) {
  int dev = 0;
  int bpw = kReindexBlocks;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && g_cus[dev] > 0) {
    const int64_t cus = g_cus[dev];
    const int64_t wgs32 = (int64_t)q->n_q * ((d->pool_blocks + kReindexBlocksNarrow - 1) / kReindexBlocksNarrow);
    const int64_t wgs64 = (int64_t)q->n_q * ((d->pool_blocks + kReindexBlocks - 1) / kReindexBlocks);
    const int64_t wgs128 = (int64_t)q->n_q * ((d->pool_blocks + kReindexBlocksWide - 1) / kReindexBlocksWide);
    bpw = wgs32 <= cus ? kReindexBlocksNarrow
        : wgs64 <= 2 * cus ? kReindexBlocks
        : wgs128 <= cus ? kReindexBlocksWide : kReindexBlocksHuge;
  }
  if (const char* env = getenv("CSA2_REINDEX_BLOCKS")) {
    const int v = atoi(env);
    if (v == kReindexBlocks || v == kReindexBlocksWide || v == kReindexBlocksNarrow || v == kReindexBlocksHuge) bpw = v;
  }
  return bpw;
}

// Marking workgroups per query: one per chunk, unless that grid would exceed
// two workgroups per CU; then as many as keep it to two per CU, each taking
// a run of chunks (256 queries with 16 chunks each: 198 us of marking with a
// workgroup per chunk, 16 rounds).  CSA2_POOL_MARK_WGS overrides (1..chunks).
// Called after check_device.
int pool_mark_wgs(const csa2_queries* q, int chunks) {
  int dev = 0;
  int wpq = chunks;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && g_cus[dev] > 0) {
    const int64_t cap = 2 * (int64_t)g_cus[dev];
    if ((int64_t)q->n_q * chunks > cap) {
      const int64_t w = cap / q->n_q;
      wpq = (int)(w < 1 ? 1 : w);
    }
  }
  if (const char* env = getenv("CSA2_POOL_MARK_WGS")) {
    const int v = atoi(env);
    if (v >= 1) wpq = v;
  }
  return wpq < chunks ? wpq : chunks;
}

struct AttendPlan { int hg, splits, split_tiles; };

// Workgroups of 32 heads; a query's tiles (the window's, then the kept
// entries', 64 each) are split so that the grid holds about one workgroup
// per CU of the 256-CU part (one tile per split when a batch has few
// queries); a second kernel merges the splits' partials.  The plan depends
// only on the sizes, so the workspace size does too.  CSA2_ATTEND_SPLITS
// overrides (1..16).
AttendPlan attend_plan(const csa2_dims* d, const csa2_queries* q) {
  AttendPlan p;
  p.hg = (d->n_heads + kAttendHeads - 1) / kAttendHeads;
  const int tiles = (d->swa + kAttendTile - 1) / kAttendTile + (d->topk + kAttendTile - 1) / kAttendTile;
  const int64_t units = (int64_t)q->n_q * p.hg;
  int s = (int)((256 + units - 1) / units);
  if (const char* env = getenv("CSA2_ATTEND_SPLITS")) s = atoi(env);
  const int cap = tiles < kAttendMaxSplits ? tiles : kAttendMaxSplits;
  s = s < 1 ? 1 : (s > cap ? cap : s);
  p.split_tiles = (tiles + s - 1) / s;
  // a split holds at most kAttendMaxTiles tiles (every query's whole list
  // fits: 1024 / 64 + 2048 / 64 = 48)
  if (p.split_tiles > kAttendMaxTiles) p.split_tiles = kAttendMaxTiles;
  p.splits = (tiles + p.split_tiles - 1) / p.split_tiles;
  return p;
}

// Attention workspace (splits > 1): the splits' partials
size_t attend_ws(const csa2_dims* d, const csa2_queries* q) {
  const AttendPlan p = attend_plan(d, q);
  if (p.splits == 1) return 0;
  const size_t rows = (size_t)q->n_q * p.splits * p.hg * kAttendHeads;
  return align256(rows * 512 * 4) + align256(rows * 2 * 4);
}

csa2_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return CSA2_OK;
  if (!ws) return fail(CSA2_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (((uintptr_t)ws) & 255) return fail(CSA2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(CSA2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return CSA2_OK;
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported device";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* csa2_last_error(void) { return g_err; }

csa2_status csa2_encode_kv(int64_t n, const uint16_t* latent, const uint16_t* rope, const int64_t* dst_row,
                           uint8_t* kv_codes, uint8_t* kv_scales, uint16_t* kv_rope, void* stream) {
  return csa2_encode_kv_grouped(n, 16, latent, rope, dst_row, kv_codes, kv_scales, kv_rope, stream);
}

csa2_status csa2_encode_kv_grouped(int64_t n, int32_t group, const uint16_t* latent, const uint16_t* rope,
                                   const int64_t* dst_row, uint8_t* kv_codes, uint8_t* kv_scales,
                                   uint16_t* kv_rope, void* stream) {
  if (group != 16 && group != 32) return fail(CSA2_ERR_INVALID_ARG, "group must be 16 or 32 (got %d)", group);
  if (n < 0) return fail(CSA2_ERR_INVALID_ARG, "n must be >= 0 (got %lld)", (long long)n);
  if (n > ((int64_t)1 << 36)) return fail(CSA2_ERR_INVALID_ARG, "n too large");
  if (n == 0) return CSA2_OK;
  if (!latent || !rope || !kv_codes || !kv_scales || !kv_rope)
    return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (((uintptr_t)latent | (uintptr_t)rope | (uintptr_t)kv_rope) & 15)
    return fail(CSA2_ERR_INVALID_ARG, "latent, rope and kv_rope must be 16-byte aligned");
  if ((uintptr_t)kv_codes & 7) return fail(CSA2_ERR_INVALID_ARG, "kv_codes must be 8-byte aligned");
  csa2_status st = check_device();
  if (st) return st;
  if (group == 32 && ((uintptr_t)kv_codes & 15)) return fail(CSA2_ERR_INVALID_ARG, "kv_codes must be 16-byte aligned");
  hipError_t e = launch_encode(n, group, latent, rope, dst_row, kv_codes, kv_scales, kv_rope, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "encode launch");
}

csa2_status csa2_encode_fp4(int64_t n, int32_t width, const uint16_t* src, const int64_t* dst_row,
                            uint8_t* codes, uint8_t* scales, void* stream) {
  if (n < 0) return fail(CSA2_ERR_INVALID_ARG, "n must be >= 0 (got %lld)", (long long)n);
  if (n > ((int64_t)1 << 36)) return fail(CSA2_ERR_INVALID_ARG, "n too large");
  if (width != 16 && width != 32 && width != 64 && width != 128 && width != 256 && width != 512 && width != 1024)
    return fail(CSA2_ERR_INVALID_ARG, "width must be 16 times a power of two, at most 1024 (got %d)", width);
  if (n == 0) return CSA2_OK;
  if (!src || !codes || !scales) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if ((uintptr_t)src & 15) return fail(CSA2_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if ((uintptr_t)codes & 7) return fail(CSA2_ERR_INVALID_ARG, "codes must be 8-byte aligned");
  csa2_status st = check_device();
  if (st) return st;
  hipError_t e = launch_encode_rows(n, width, src, dst_row, codes, scales, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "encode launch");
}

csa2_status csa2_index_full_workspace_size(const csa2_dims* d, const csa2_queries* q, size_t* bytes) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!bytes) return fail(CSA2_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = full_ws(d, q);
  return CSA2_OK;
}

static csa2_status check_block_scores(const csa2_dims* d, const csa2_queries* q, const float* block_scores,
                                      int64_t ld_block_scores) {
  // at least 4 even with no blocks: the pool select's clamped 16-byte loads
  // read inside [0, ld) of every row
  const int64_t nb = max_blocks(d, q);
  if (ld_block_scores < nb || ld_block_scores < 4)
    return fail(CSA2_ERR_INVALID_ARG, "ld_block_scores %lld < max(4, %lld blocks)", (long long)ld_block_scores,
                (long long)nb);
  if ((ld_block_scores & 3) || ((uintptr_t)block_scores & 15))
    return fail(CSA2_ERR_INVALID_ARG, "block_scores must be 16-byte aligned with ld_block_scores a multiple of 4");
  return CSA2_OK;
}

// Position keys: a multiple of 32 per row, covering every candidate position
// rounded up to 32 (the scan writes whole 16-position steps), 16-byte aligned.
static csa2_status check_pos_keys(const csa2_dims* d, const csa2_queries* q, const uint32_t* pkey, int64_t ld) {
  const int64_t need = (max_blocks(d, q) * 8 + 31) / 32 * 32;
  if (ld < need || ld % 32 || ((uintptr_t)pkey & 15))
    return fail(CSA2_ERR_INVALID_ARG, "pos_keys: ld_pos_keys %lld must be a multiple of 32 >= %lld, 16-byte aligned",
                (long long)ld, (long long)need);
  return CSA2_OK;
}

// The Full scan; with pool_ws it also leaves the per-tile key ranges and a
// cleared histogram for the pool select.
static csa2_status run_scan(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const uint8_t* q_scales,
                            const float* idx_w, const uint8_t* idx_k, const uint8_t* k_scales, float* block_scores,
                            int64_t ld_block_scores, uint32_t* pool_ws_ptr, void* stream,
                            const csa2_pages* pages = nullptr, uint32_t* pkey = nullptr, int64_t ld_pkey = 0) {
  ScanArgs sa;
  sa.idx_q = idx_q; sa.idx_w = idx_w; sa.idx_k = idx_k;
  sa.idx_q_scales = q_scales; sa.idx_k_scales = k_scales;
  sa.seq_base = q->seq_base; sa.n_visible = q->n_visible;
  sa.n_q = q->n_q; sa.hi = d->idx_heads; sa.d = d->idx_dim; sa.swa = d->swa; sa.g = q->tokens_per_seq;
  int pf = kScanPrefetch, nw = kScanWaves;
  if (const char* env = getenv("CSA2_SCAN_PREFETCH")) pf = atoi(env);
  if (const char* env = getenv("CSA2_SCAN_WAVES")) nw = atoi(env);
  if (pf != 4 && pf != 6 && pf != 8) pf = kScanPrefetch;
  if (nw != 4 && nw != 8) nw = kScanWaves;
  sa.tile_pos = scan_tile(d, q);
  sa.prefetch = pf;
  sa.waves = nw;
  sa.tiles = scan_tiles(d, q, sa.tile_pos);
  sa.tile_extra = scan_tile_extra(d, q, sa.tile_pos, sa.tiles);
  sa.bscore = block_scores;
  sa.ld = ld_block_scores;
  sa.pool_ws = pool_ws_ptr;
  sa.pool_ws_stride = pool_ws_words(pool_chunks(d, q), pool_mm_cap(d, q));
  sa.pages = pages ? pages->table : nullptr;
  sa.page_shift = pages ? page_shift(pages) : 0;
  sa.rows = pages ? pages->rows : 0;
  sa.pkey = pkey;
  sa.ld_pkey = ld_pkey;
  sa.gkey = nullptr;
  sa.ld_gkey = 0;
  if (pool_ws_ptr && scan_groups_ok(d, q)) {
    sa.gkey = pool_ws_ptr + pool_gkey_off(pool_chunks(d, q), pool_mm_cap(d, q));
    sa.ld_gkey = sa.pool_ws_stride;
  }
  hipError_t e = launch_scan(sa, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "scan launch");
}

// With topk_pos, the Full layer's Top-K from the scan's position keys follows
// the pool: inside the selecting workgroup for small pools, else by
// k_topk_keys after the chunked kernels.
static csa2_status run_pool(const csa2_dims* d, const csa2_queries* q, const float* block_scores, int64_t ld_block_scores,
                            int32_t* pool_blocks, int32_t* pool_count, void* ws, bool after_scan, void* stream,
                            const uint32_t* pkey = nullptr, int64_t ld_pkey = 0, int32_t* topk_pos = nullptr,
                            int32_t* topk_count = nullptr) {
  PoolArgs pa;
  pa.bscore = block_scores; pa.ld = ld_block_scores; pa.n_visible = q->n_visible;
  pa.n_q = q->n_q; pa.swa = d->swa; pa.pool = d->pool_blocks;
  pa.chunks = pool_chunks(d, q);
  pa.mark_wgs = pool_mark_wgs(q, pa.chunks);
  pa.mm_cap = pool_mm_cap(d, q);
  pa.nw_cap = (int)((max_blocks(d, q) + 31) / 32);
  pa.small = max_blocks(d, q) <= kPoolSmallBlocks;
  if (const char* env = getenv("CSA2_POOL_SMALL")) pa.small = pa.small && atoi(env) != 0;
  pa.ws = (uint32_t*)ws;
  pa.ws_stride = pool_ws_words(pa.chunks, pa.mm_cap);
  pa.have_minmax = after_scan;
  pa.mm_half = 0;
  pa.mm_span = after_scan ? scan_tile(d, q) / 8 : kPoolChunk;
  if (after_scan) {
    // the scan's tiles: the first half longer when it split them unevenly
    const int tile = scan_tile(d, q), tiles = scan_tiles(d, q, tile);
    const int extra = scan_tile_extra(d, q, tile, tiles);
    if (extra) {
      pa.mm_half = tiles / 2;
      pa.mm_span = (tile - extra) / 8;
    }
    pa.mm_span1 = (tile + extra) / 8;
  } else {
    pa.mm_span1 = pa.mm_span;
  }
  pa.pool_blocks = pool_blocks; pa.pool_count = pool_count;
  const bool fused = topk_pos && pa.small;
  pa.pkey = fused ? pkey : nullptr; pa.ld_pkey = ld_pkey; pa.topk = d->topk;
  pa.topk_pos = fused ? topk_pos : nullptr; pa.topk_count = fused ? topk_count : nullptr;
  hipError_t e = launch_pool_select(pa, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool select launch");
  if (topk_pos && !fused) {
    TopkKeysArgs ta;
    ta.pool_blocks = pool_blocks; ta.pool_count = pool_count;
    ta.bscore = block_scores; ta.ld = ld_block_scores;
    ta.pkey = pkey; ta.ld_pkey = ld_pkey;
    ta.n_q = q->n_q; ta.pool = d->pool_blocks; ta.topk = d->topk;
    ta.topk_pos = topk_pos; ta.topk_count = topk_count; ta.topk_scores = nullptr;
    e = launch_topk_keys(ta, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
  }
  return CSA2_OK;
}

// The indexer rows of a call: fp8 (no scale planes) or FP4 (both planes).
static csa2_status check_index_rows(const csa2_dims* d, const uint8_t* idx_q, const uint8_t* q_scales, const float* idx_w,
                                    const uint8_t* idx_k, const uint8_t* k_scales, bool fp4) {
  if (!idx_q || !idx_w || !idx_k) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (((uintptr_t)idx_q | (uintptr_t)idx_k) & 15)
    return fail(CSA2_ERR_INVALID_ARG, "query and key rows must be 16-byte aligned");
  if (fp4) {
    if (!q_scales || !k_scales) return fail(CSA2_ERR_INVALID_ARG, "FP4 scale pointer is NULL");
    if (((uintptr_t)q_scales | (uintptr_t)k_scales) & 7)
      return fail(CSA2_ERR_INVALID_ARG, "FP4 scale planes must be 8-byte aligned");
    if (d->idx_dim != 128) return fail(CSA2_ERR_INVALID_ARG, "FP4 indexer rows need idx_dim 128 (got %d)", d->idx_dim);
  }
  return CSA2_OK;
}

static csa2_status index_scan(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const uint8_t* q_scales,
                              const float* idx_w, const uint8_t* idx_k, const uint8_t* k_scales, bool fp4,
                              float* block_scores, int64_t ld_block_scores, void* pool_wsp, size_t pool_ws_bytes,
                              void* stream, const csa2_pages* pages = nullptr, uint32_t* pkey = nullptr,
                              int64_t ld_pkey = 0) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if ((st = check_index_rows(d, idx_q, q_scales, idx_w, idx_k, k_scales, fp4))) return st;
  if (pages && (st = check_pages(pages, fp4 ? d->idx_dim / 2 : d->idx_dim))) return st;
  if (!block_scores) return fail(CSA2_ERR_INVALID_ARG, "block_scores is NULL");
  if ((st = check_block_scores(d, q, block_scores, ld_block_scores))) return st;
  if (pool_wsp && (st = check_ws(pool_wsp, pool_ws_bytes, pool_ws(d, q)))) return st;
  if (pkey && (st = check_pos_keys(d, q, pkey, ld_pkey))) return st;
  if ((st = check_device())) return st;
  return run_scan(d, q, idx_q, fp4 ? q_scales : nullptr, idx_w, idx_k, fp4 ? k_scales : nullptr, block_scores,
                  ld_block_scores, (uint32_t*)pool_wsp, stream, pages, pkey, ld_pkey);
}

csa2_status csa2_index_scan_keys(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                 const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                 const uint8_t* idx_k, const uint8_t* idx_k_scales, float* block_scores,
                                 int64_t ld_block_scores, uint32_t* pos_keys, int64_t ld_pos_keys, void* pool_wsp,
                                 size_t pool_ws_bytes, void* stream) {
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  if (!pos_keys) return fail(CSA2_ERR_INVALID_ARG, "pos_keys is NULL");
  return index_scan(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, idx_q_scales != nullptr, block_scores,
                    ld_block_scores, pool_wsp, pool_ws_bytes, stream, pages, pos_keys, ld_pos_keys);
}

csa2_status csa2_index_topk_keys(const csa2_dims* d, const csa2_queries* q, const int32_t* pool_blocks,
                                 const int32_t* pool_count, const float* block_scores, int64_t ld_block_scores,
                                 const uint32_t* pos_keys, int64_t ld_pos_keys, int32_t* topk_pos,
                                 int32_t* topk_count, float* topk_scores, void* stream) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!pool_blocks || !pool_count || !block_scores || !pos_keys || !topk_pos || !topk_count)
    return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if ((st = check_block_scores(d, q, block_scores, ld_block_scores))) return st;
  if ((st = check_pos_keys(d, q, pos_keys, ld_pos_keys))) return st;
  if ((st = check_device())) return st;
  TopkKeysArgs ta;
  ta.pool_blocks = pool_blocks; ta.pool_count = pool_count;
  ta.bscore = block_scores; ta.ld = ld_block_scores;
  ta.pkey = pos_keys; ta.ld_pkey = ld_pos_keys;
  ta.n_q = q->n_q; ta.pool = d->pool_blocks; ta.topk = d->topk;
  ta.topk_pos = topk_pos; ta.topk_count = topk_count; ta.topk_scores = topk_scores;
  hipError_t e = launch_topk_keys(ta, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "top-k launch");
}

csa2_status csa2_index_scan_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                  const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                  const uint8_t* idx_k, const uint8_t* idx_k_scales, float* block_scores,
                                  int64_t ld_block_scores, void* pool_wsp, size_t pool_ws_bytes, void* stream) {
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return index_scan(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, idx_q_scales != nullptr, block_scores,
                    ld_block_scores, pool_wsp, pool_ws_bytes, stream, pages);
}

csa2_status csa2_index_scan(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const float* idx_w,
                            const uint8_t* idx_k, float* block_scores, int64_t ld_block_scores, void* pool_wsp,
                            size_t pool_ws_bytes, void* stream) {
  return index_scan(d, q, idx_q, nullptr, idx_w, idx_k, nullptr, false, block_scores, ld_block_scores, pool_wsp,
                    pool_ws_bytes, stream);
}

csa2_status csa2_index_scan_fp4(const csa2_dims* d, const csa2_queries* q, const uint8_t* q_codes,
                                const uint8_t* q_scales, const float* idx_w, const uint8_t* k_codes,
                                const uint8_t* k_scales, float* block_scores, int64_t ld_block_scores,
                                void* pool_wsp, size_t pool_ws_bytes, void* stream) {
  return index_scan(d, q, q_codes, q_scales, idx_w, k_codes, k_scales, true, block_scores, ld_block_scores,
                    pool_wsp, pool_ws_bytes, stream);
}

csa2_status csa2_index_pool_workspace_size(const csa2_dims* d, const csa2_queries* q, size_t* bytes) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!bytes) return fail(CSA2_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = pool_ws(d, q);
  return CSA2_OK;
}

csa2_status csa2_index_pool(const csa2_dims* d, const csa2_queries* q, const float* block_scores,
                            int64_t ld_block_scores, int32_t* pool_blocks, int32_t* pool_count, void* ws,
                            size_t ws_bytes, int32_t flags, void* stream) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!block_scores || !pool_blocks || !pool_count) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (flags & ~CSA2_POOL_WS_FROM_SCAN) return fail(CSA2_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((st = check_block_scores(d, q, block_scores, ld_block_scores))) return st;
  if ((st = check_ws(ws, ws_bytes, pool_ws(d, q)))) return st;
  if ((st = check_device())) return st;
  return run_pool(d, q, block_scores, ld_block_scores, pool_blocks, pool_count, ws,
                  (flags & CSA2_POOL_WS_FROM_SCAN) != 0, stream);
}

csa2_status csa2_index_pool_topk(const csa2_dims* d, const csa2_queries* q, const float* block_scores,
                                 int64_t ld_block_scores, const uint32_t* pos_keys, int64_t ld_pos_keys,
                                 int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                 void* ws, size_t ws_bytes, int32_t flags, void* stream) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!block_scores || !pool_blocks || !pool_count || !pos_keys || !topk_pos || !topk_count)
    return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (flags & ~CSA2_POOL_WS_FROM_SCAN) return fail(CSA2_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((st = check_block_scores(d, q, block_scores, ld_block_scores))) return st;
  if ((st = check_pos_keys(d, q, pos_keys, ld_pos_keys))) return st;
  if ((st = check_ws(ws, ws_bytes, pool_ws(d, q)))) return st;
  if ((st = check_device())) return st;
  return run_pool(d, q, block_scores, ld_block_scores, pool_blocks, pool_count, ws,
                  (flags & CSA2_POOL_WS_FROM_SCAN) != 0, stream, pos_keys, ld_pos_keys, topk_pos, topk_count);
}

static csa2_status index_full(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const uint8_t* q_scales,
                              const float* idx_w, const uint8_t* idx_k, const uint8_t* k_scales, bool fp4,
                              int32_t* pool_blocks, int32_t* pool_count, float* block_scores, int64_t ld_block_scores,
                              void* ws, size_t ws_bytes, void* stream, bool dry = false,
                              const csa2_pages* pages = nullptr, uint32_t* pkey = nullptr,
                              int32_t* topk_pos = nullptr, int32_t* topk_count = nullptr, bool scan_only = false) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if ((st = check_index_rows(d, idx_q, q_scales, idx_w, idx_k, k_scales, fp4))) return st;
  if (pages && (st = check_pages(pages, fp4 ? d->idx_dim / 2 : d->idx_dim))) return st;
  if (!pool_blocks || !pool_count) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  const size_t pw = pool_ws(d, q);
  if ((st = check_ws(ws, ws_bytes, block_scores ? pw : full_ws(d, q)))) return st;
  float* bs = block_scores;
  int64_t ld = ld_block_scores;
  if (!bs) {
    bs = (float*)((char*)ws + pw);
    ld = full_ldb(d, q);
  }
  if ((st = check_block_scores(d, q, bs, ld))) return st;
  if ((st = check_device())) return st;
  if (dry) return CSA2_OK;
  if ((st = run_scan(d, q, idx_q, fp4 ? q_scales : nullptr, idx_w, idx_k, fp4 ? k_scales : nullptr, bs, ld,
                     (uint32_t*)ws, stream, pages, pkey, pkey ? full_ldpk(d, q) : 0)))
    return st;
  if (scan_only) return CSA2_OK;
  return run_pool(d, q, bs, ld, pool_blocks, pool_count, ws, true, stream, pkey, pkey ? full_ldpk(d, q) : 0,
                  pkey ? topk_pos : nullptr, pkey ? topk_count : nullptr);
}

csa2_status csa2_index_full(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const float* idx_w,
                            const uint8_t* idx_k, int32_t* pool_blocks, int32_t* pool_count, float* block_scores,
                            int64_t ld_block_scores, void* ws, size_t ws_bytes, void* stream) {
  return index_full(d, q, idx_q, nullptr, idx_w, idx_k, nullptr, false, pool_blocks, pool_count, block_scores,
                    ld_block_scores, ws, ws_bytes, stream);
}

csa2_status csa2_index_full_fp4(const csa2_dims* d, const csa2_queries* q, const uint8_t* q_codes,
                                const uint8_t* q_scales, const float* idx_w, const uint8_t* k_codes,
                                const uint8_t* k_scales, int32_t* pool_blocks, int32_t* pool_count,
                                float* block_scores, int64_t ld_block_scores, void* ws, size_t ws_bytes,
                                void* stream) {
  return index_full(d, q, q_codes, q_scales, idx_w, k_codes, k_scales, true, pool_blocks, pool_count, block_scores,
                    ld_block_scores, ws, ws_bytes, stream);
}

csa2_status csa2_index_full_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                  const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                  const uint8_t* idx_k, const uint8_t* idx_k_scales, int32_t* pool_blocks,
                                  int32_t* pool_count, float* block_scores, int64_t ld_block_scores, void* ws,
                                  size_t ws_bytes, void* stream) {
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return index_full(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, idx_q_scales != nullptr, pool_blocks,
                    pool_count, block_scores, ld_block_scores, ws, ws_bytes, stream, false, pages);
}

csa2_status csa2_index_reindex_workspace_size(const csa2_dims* d, const csa2_queries* q, size_t* bytes) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!bytes) return fail(CSA2_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = reindex_ws(d, q);
  return CSA2_OK;
}

// counters: when given, the per-query completion counters live there (zero
// between calls) and ws holds only the order keys
static csa2_status index_reindex(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const uint8_t* q_scales,
                                 const float* idx_w, const uint8_t* idx_k, const uint8_t* k_scales, bool fp4,
                                 const int32_t* pool_blocks, const int32_t* pool_count, int32_t* topk_pos,
                                 int32_t* topk_count, float* topk_scores, void* ws, size_t ws_bytes, void* stream,
                                 bool dry = false, const csa2_pages* pages = nullptr, uint32_t* counters = nullptr,
                                 bool score_only = false) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if ((st = check_index_rows(d, idx_q, q_scales, idx_w, idx_k, k_scales, fp4))) return st;
  if (pages && (st = check_pages(pages, fp4 ? d->idx_dim / 2 : d->idx_dim))) return st;
  if (!pool_blocks || !pool_count || !topk_pos || !topk_count)
    return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if ((st = check_ws(ws, ws_bytes, counters ? reindex_keys_ws(d, q) : reindex_ws(d, q)))) return st;
  if ((st = check_device())) return st;
  if (dry) return CSA2_OK;
  ReindexArgs ra;
  ra.idx_q = idx_q; ra.idx_w = idx_w; ra.idx_k = idx_k;
  ra.idx_q_scales = fp4 ? q_scales : nullptr;
  ra.idx_k_scales = fp4 ? k_scales : nullptr;
  ra.seq_base = q->seq_base; ra.n_visible = q->n_visible;
  ra.pool_blocks = pool_blocks; ra.pool_count = pool_count;
  ra.n_q = q->n_q; ra.hi = d->idx_heads; ra.d = d->idx_dim; ra.swa = d->swa;
  ra.pool = d->pool_blocks; ra.topk = d->topk;
  ra.blocks_per_wg = reindex_blocks_per_wg(d, q);
  ra.split = (d->pool_blocks + ra.blocks_per_wg - 1) / ra.blocks_per_wg;
  ra.done = counters ? counters : (uint32_t*)ws;
  ra.keys = counters ? (uint32_t*)ws : (uint32_t*)((char*)ws + align256((size_t)q->n_q * 4));
  ra.topk_pos = topk_pos; ra.topk_count = topk_count; ra.topk_scores = topk_scores;
  ra.score_only = score_only ? 1 : 0;
  ra.pages = pages ? pages->table : nullptr;
  ra.page_shift = pages ? page_shift(pages) : 0;
  ra.rows = pages ? pages->rows : 0;
  hipError_t e = launch_reindex(ra, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "reindex launch");
}

csa2_status csa2_index_reindex(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q, const float* idx_w,
                               const uint8_t* idx_k, const int32_t* pool_blocks, const int32_t* pool_count,
                               int32_t* topk_pos, int32_t* topk_count, float* topk_scores, void* ws,
                               size_t ws_bytes, void* stream) {
  return index_reindex(d, q, idx_q, nullptr, idx_w, idx_k, nullptr, false, pool_blocks, pool_count, topk_pos,
                       topk_count, topk_scores, ws, ws_bytes, stream);
}

csa2_status csa2_index_reindex_fp4(const csa2_dims* d, const csa2_queries* q, const uint8_t* q_codes,
                                   const uint8_t* q_scales, const float* idx_w, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const int32_t* pool_blocks, const int32_t* pool_count,
                                   int32_t* topk_pos, int32_t* topk_count, float* topk_scores, void* ws,
                                   size_t ws_bytes, void* stream) {
  return index_reindex(d, q, q_codes, q_scales, idx_w, k_codes, k_scales, true, pool_blocks, pool_count, topk_pos,
                       topk_count, topk_scores, ws, ws_bytes, stream);
}

csa2_status csa2_index_reindex_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                     const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                     const uint8_t* idx_k, const uint8_t* idx_k_scales, const int32_t* pool_blocks,
                                     const int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                     float* topk_scores, void* ws, size_t ws_bytes, void* stream) {
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return index_reindex(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, idx_q_scales != nullptr, pool_blocks,
                       pool_count, topk_pos, topk_count, topk_scores, ws, ws_bytes, stream, false, pages);
}

csa2_status csa2_attend_workspace_size(const csa2_dims* d, const csa2_queries* q, size_t* bytes) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!bytes) return fail(CSA2_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = attend_ws(d, q);
  return CSA2_OK;
}

// The pool and the Full layer's Top-K selected inside the attention kernel
// (csa2_pool_topk_attend): the scan's scores in, the selection out.
struct AttendSel {
  const float* block_scores;
  int64_t ld_block_scores;
  const uint32_t* pos_keys;
  int64_t ld_pos_keys;
  int32_t* pool_blocks;
  int32_t* pool_count;
  bool from_pool;            // the pool is selected before (chunked kernels): only the Top-K in the kernel
  const uint32_t* rkeys;     // Reindex order keys: the Top-K from them (block_scores, pos_keys unused)
  const uint32_t* gkeys;     // the scan's group keys: queries past kPoolSmallBlocks blocks select from them
  int64_t ld_gkeys;
  int gcap;
  int group_min;             // (and the Top-K of queries past this many blocks)
};

// Whether every query's pool fits one selecting workgroup (and the
// chunked kernels are not forced with CSA2_POOL_SMALL=0).
static bool pool_small(const csa2_dims* d, const csa2_queries* q) {
  bool small = max_blocks(d, q) <= kPoolSmallBlocks;
  if (const char* env = getenv("CSA2_POOL_SMALL")) small = small && atoi(env) != 0;
  return small;
}

static csa2_status attend(const csa2_dims* d, const csa2_queries* q, const uint16_t* q_lat, const uint16_t* q_rope,
                          float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                          const uint16_t* kv_rope, const int32_t* topk_pos, const int32_t* topk_count,
                          const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream, bool dry = false, const csa2_pages* pages = nullptr,
                          const AttendSel* sel = nullptr) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (pages && (st = check_pages(pages, 256))) return st;   // kv_codes: the widest plane
  if (sel && sel->rkeys) {
    if (!sel->pool_blocks || !sel->pool_count) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  } else if (sel) {
    if (!sel->from_pool && !sel->gkeys && !pool_small(d, q))
      return fail(CSA2_ERR_UNSUPPORTED, "the in-kernel selection takes at most %d blocks per query (max_visible %lld)",
                  kPoolSmallBlocks, (long long)q->max_visible);
    if (sel->gkeys && (max_blocks(d, q) > (int64_t)kPoolGroupsMax * kGroupBlocks || d->topk > 1024))
      return fail(CSA2_ERR_UNSUPPORTED, "the group-key selection takes at most %d blocks per query and a Top-K of 1024",
                  kPoolGroupsMax * kGroupBlocks);
    if (!sel->block_scores || !sel->pos_keys || !sel->pool_blocks || !sel->pool_count)
      return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
    if ((st = check_block_scores(d, q, sel->block_scores, sel->ld_block_scores))) return st;
    if ((st = check_pos_keys(d, q, sel->pos_keys, sel->ld_pos_keys))) return st;
  }
  if (!q_lat || !q_rope || !kv_codes || !kv_scales || !kv_rope || !topk_pos || !topk_count || !swa_base || !out)
    return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (!swa_kv && d->swa > 0) return fail(CSA2_ERR_INVALID_ARG, "swa_kv is NULL");
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return fail(CSA2_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (((uintptr_t)q_lat | (uintptr_t)q_rope | (uintptr_t)kv_rope | (uintptr_t)swa_kv | (uintptr_t)out) & 15)
    return fail(CSA2_ERR_INVALID_ARG, "q_lat, q_rope, kv_rope, swa_kv and out must be 16-byte aligned");
  if ((uintptr_t)kv_codes & 7) return fail(CSA2_ERR_INVALID_ARG, "kv_codes must be 8-byte aligned");
  if ((st = check_ws(ws, ws_bytes, attend_ws(d, q)))) return st;
  if ((st = check_device())) return st;
  if (dry) return CSA2_OK;
  const AttendPlan p = attend_plan(d, q);
  AttendArgs aa;
  aa.q_lat = q_lat; aa.q_rope = q_rope; aa.scale_log2 = softmax_scale * 1.4426950408889634f;
  aa.kv_codes = kv_codes; aa.kv_scales = kv_scales; aa.kv_rope = kv_rope;
  aa.kv_gshift = d->kv_group == 32 ? 1 : 0;
  aa.topk_pos = topk_pos; aa.topk_count = topk_count; aa.swa_kv = swa_kv; aa.swa_base = swa_base;
  aa.seq_base = q->seq_base; aa.n_visible = q->n_visible;
  aa.n_q = q->n_q; aa.heads = d->n_heads; aa.topk = d->topk; aa.swa = d->swa;
  aa.head_groups = p.hg; aa.splits = p.splits; aa.split_tiles = p.split_tiles;
  aa.out = out; aa.lse = lse;
  aa.pages = pages ? pages->table : nullptr;
  aa.page_shift = pages ? page_shift(pages) : 0;
  aa.rows = pages ? pages->rows : 0;
  aa.part_o = nullptr; aa.part_ml = nullptr;
  aa.bscore = nullptr; aa.ld_bs = 0; aa.pkey = nullptr; aa.ld_pkey = 0; aa.pool = d->pool_blocks;
  aa.pool_blocks = nullptr; aa.pool_count = nullptr; aa.topk_out = nullptr; aa.topk_count_out = nullptr;
  aa.sel_from_pool = 0;
  aa.rkeys = nullptr;
  aa.gkey = nullptr; aa.ld_gkey = 0; aa.gcap = 0; aa.group_min = kPoolSmallBlocks;
  if (sel) {
    aa.sel_from_pool = sel->from_pool ? 1 : 0;
    aa.rkeys = sel->rkeys;
    aa.gkey = sel->gkeys; aa.ld_gkey = sel->ld_gkeys; aa.gcap = sel->gcap; aa.group_min = sel->group_min;
    aa.bscore = sel->block_scores; aa.ld_bs = sel->ld_block_scores;
    aa.pkey = sel->pos_keys; aa.ld_pkey = sel->ld_pos_keys;
    aa.pool_blocks = sel->pool_blocks; aa.pool_count = sel->pool_count;
    aa.topk_out = const_cast<int32_t*>(topk_pos); aa.topk_count_out = const_cast<int32_t*>(topk_count);
    aa.topk_pos = nullptr; aa.topk_count = nullptr;
  }
  if (p.splits > 1) {
    const size_t rows = (size_t)q->n_q * p.splits * p.hg * kAttendHeads;
    aa.part_o = (float*)ws;
    aa.part_ml = (float*)((char*)ws + align256(rows * 512 * 4));
  }
  hipError_t e = launch_attend(aa, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "attend launch");
}

csa2_status csa2_attend(const csa2_dims* d, const csa2_queries* q, const uint16_t* q_lat, const uint16_t* q_rope,
                        float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                        const uint16_t* kv_rope, const int32_t* topk_pos, const int32_t* topk_count,
                        const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse, void* ws,
                        size_t ws_bytes, void* stream) {
  return attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                swa_base, out, lse, ws, ws_bytes, stream);
}

csa2_status csa2_attend_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                              const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                              const int32_t* topk_pos, const int32_t* topk_count, const uint16_t* swa_kv,
                              const int64_t* swa_base, float* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                swa_base, out, lse, ws, ws_bytes, stream, false, pages);
}

// The pool and the Full layer's Top-K with the attention on it: for small
// pools one attention launch that selects both; otherwise the chunked pool
// kernels, then the attention launch that selects the Top-K of that pool.
static csa2_status pool_topk_attend(const csa2_dims* d, const csa2_queries* q, const float* block_scores,
                                    int64_t ld_block_scores, const uint32_t* pos_keys, int64_t ld_pos_keys,
                                    int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                    const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                                    const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                                    const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                                    void* pool_wsp, size_t pool_ws_bytes, int32_t flags, void* ws, size_t ws_bytes,
                                    void* stream, bool dry = false, const csa2_pages* pages = nullptr) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (flags & ~CSA2_POOL_WS_FROM_SCAN) return fail(CSA2_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool small = pool_small(d, q);
  if ((st = check_device())) return st;          // (the scan's tile shape reads the device)
  // a long query after the scan: pool and Top-K from the scan's group keys
  // in the attention launch (CSA2_POOL_GROUPS=0: the chunked pool kernels)
  // (CSA2_GROUP_MIN: the Top-K of queries past that many blocks from the
  // group keys too, small pools included; for tuning)
  int group_min = kPoolSmallBlocks;
  if (const char* env = getenv("CSA2_GROUP_MIN")) group_min = std::min(std::max(atoi(env), 0), kPoolSmallBlocks);
  bool groups = (!small || (group_min < kPoolSmallBlocks && pool_wsp)) && (flags & CSA2_POOL_WS_FROM_SCAN) &&
                scan_groups_ok(d, q) && max_blocks(d, q) <= (int64_t)kPoolGroupsMax * kGroupBlocks &&
                d->topk <= 1024 && d->topk <= d->pool_blocks && 2 * d->pool_blocks <= 4096;   // (K > P: the exact pool decides)
  if (const char* env = getenv("CSA2_POOL_GROUPS")) groups = groups && atoi(env) != 0;
  if ((!small || groups) && (st = check_ws(pool_wsp, pool_ws_bytes, pool_ws(d, q)))) return st;
  // a Top-K of more than 1024 positions from a given pool is selected apart
  // (k_topk_keys): its positions step does not fit beside the attention
  const bool apart = !small && !groups && d->topk > 1024;
  if (!block_scores || !pos_keys) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (apart && ((st = check_block_scores(d, q, block_scores, ld_block_scores)) ||
                (st = check_pos_keys(d, q, pos_keys, ld_pos_keys))))
    return st;
  AttendSel sel{block_scores, ld_block_scores, pos_keys, ld_pos_keys, pool_blocks, pool_count, !small && !groups,
                nullptr, nullptr, 0, 0, group_min};
  if (groups) {
    sel.gkeys = (const uint32_t*)pool_wsp + pool_gkey_off(pool_chunks(d, q), pool_mm_cap(d, q));
    sel.ld_gkeys = pool_ws_words(pool_chunks(d, q), pool_mm_cap(d, q));
    sel.gcap = pool_gcap(d, q);
  }
  // every argument is checked before the first launch
  if ((st = attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                   swa_base, out, lse, ws, ws_bytes, stream, true, pages, apart ? nullptr : &sel)))
    return st;
  if (dry) return CSA2_OK;
  if (!small && !groups && (st = run_pool(d, q, block_scores, ld_block_scores, pool_blocks, pool_count, pool_wsp,
                               (flags & CSA2_POOL_WS_FROM_SCAN) != 0, stream, pos_keys, ld_pos_keys,
                               apart ? topk_pos : nullptr, apart ? topk_count : nullptr)))
    return st;
  return attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                swa_base, out, lse, ws, ws_bytes, stream, false, pages, apart ? nullptr : &sel);
}

csa2_status csa2_pool_topk_attend(const csa2_dims* d, const csa2_queries* q, const float* block_scores,
                                  int64_t ld_block_scores, const uint32_t* pos_keys, int64_t ld_pos_keys,
                                  int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                  const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                                  const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                                  const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                                  void* pool_ws, size_t pool_ws_bytes, int32_t flags, void* ws, size_t ws_bytes,
                                  void* stream) {
  return pool_topk_attend(d, q, block_scores, ld_block_scores, pos_keys, ld_pos_keys, pool_blocks, pool_count,
                          topk_pos, topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv,
                          swa_base, out, lse, pool_ws, pool_ws_bytes, flags, ws, ws_bytes, stream);
}

csa2_status csa2_pool_topk_attend_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                        const float* block_scores, int64_t ld_block_scores, const uint32_t* pos_keys,
                                        int64_t ld_pos_keys, int32_t* pool_blocks, int32_t* pool_count,
                                        int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat,
                                        const uint16_t* q_rope, float softmax_scale, const uint8_t* kv_codes,
                                        const uint8_t* kv_scales, const uint16_t* kv_rope, const uint16_t* swa_kv,
                                        const int64_t* swa_base, float* out, float* lse, void* pool_ws,
                                        size_t pool_ws_bytes, int32_t flags, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return pool_topk_attend(d, q, block_scores, ld_block_scores, pos_keys, ld_pos_keys, pool_blocks, pool_count,
                          topk_pos, topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv,
                          swa_base, out, lse, pool_ws, pool_ws_bytes, flags, ws, ws_bytes, stream, false, pages);
}

// A Reindex layer: the scoring kernel writes the order keys only, and the
// attention workgroups select the Top-K from them.
static csa2_status reindex_attend(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q,
                                  const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                                  const uint8_t* idx_k_scales, const int32_t* pool_blocks, const int32_t* pool_count,
                                  int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat,
                                  const uint16_t* q_rope, float softmax_scale, const uint8_t* kv_codes,
                                  const uint8_t* kv_scales, const uint16_t* kv_rope, const uint16_t* swa_kv,
                                  const int64_t* swa_base, float* out, float* lse, void* reindex_wsp,
                                  size_t reindex_ws_bytes, void* ws, size_t ws_bytes, void* stream, bool dry = false,
                                  uint32_t* counters = nullptr, const csa2_pages* pages = nullptr) {
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  const bool fp4 = idx_q_scales != nullptr;
  csa2_status st;
  if ((st = index_reindex(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, fp4, pool_blocks, pool_count,
                          topk_pos, topk_count, nullptr, reindex_wsp, reindex_ws_bytes, stream, true, pages,
                          counters, true)))
    return st;
  // the keys sit after the completion counters (or at the start, with
  // external counters)
  const uint32_t* rkeys = counters ? (const uint32_t*)reindex_wsp
                                   : (const uint32_t*)((const char*)reindex_wsp + align256((size_t)q->n_q * 4));
  const AttendSel sel{nullptr, 0, nullptr, 0, const_cast<int32_t*>(pool_blocks), const_cast<int32_t*>(pool_count),
                      true, rkeys};
  if ((st = attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                   swa_base, out, lse, ws, ws_bytes, stream, true, pages, &sel)))
    return st;
  if (dry) return CSA2_OK;
  if ((st = index_reindex(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, fp4, pool_blocks, pool_count,
                          topk_pos, topk_count, nullptr, reindex_wsp, reindex_ws_bytes, stream, false, pages,
                          counters, true)))
    return st;
  return attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                swa_base, out, lse, ws, ws_bytes, stream, false, pages, &sel);
}

csa2_status csa2_reindex_attend(const csa2_dims* d, const csa2_queries* q, const uint8_t* idx_q,
                                const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                                const uint8_t* idx_k_scales, const int32_t* pool_blocks, const int32_t* pool_count,
                                int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                                float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base, float* out,
                                float* lse, void* reindex_ws, size_t reindex_ws_bytes, void* ws, size_t ws_bytes,
                                void* stream) {
  return reindex_attend(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count, topk_pos,
                        topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out,
                        lse, reindex_ws, reindex_ws_bytes, ws, ws_bytes, stream);
}

csa2_status csa2_reindex_attend_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                      const uint8_t* idx_q, const uint8_t* idx_q_scales, const float* idx_w,
                                      const uint8_t* idx_k, const uint8_t* idx_k_scales, const int32_t* pool_blocks,
                                      const int32_t* pool_count, int32_t* topk_pos, int32_t* topk_count,
                                      const uint16_t* q_lat, const uint16_t* q_rope, float softmax_scale,
                                      const uint8_t* kv_codes, const uint8_t* kv_scales, const uint16_t* kv_rope,
                                      const uint16_t* swa_kv, const int64_t* swa_base, float* out, float* lse,
                                      void* reindex_ws, size_t reindex_ws_bytes, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return reindex_attend(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count, topk_pos,
                        topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out,
                        lse, reindex_ws, reindex_ws_bytes, ws, ws_bytes, stream, false, nullptr, pages);
}

csa2_status csa2_page_rows(const csa2_pages* pages, int64_t n, const int64_t* table_off, const int32_t* pos,
                           int64_t* dst_row, void* stream) {
  csa2_status st = check_pages(pages, 1);
  if (st) return st;
  if (n < 0) return fail(CSA2_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!table_off || !pos || !dst_row)) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if ((st = check_device())) return st;
  hipError_t e = launch_page_rows(n, pages->table, page_shift(pages), table_off, pos, dst_row, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "page rows launch");
}

// ---------------------------------------------------------------- no-alloc step
// csa2_decode_step_noalloc's scratch: one array per GPU, for callers that
// cannot allocate.  Its first kScratchCounterBytes hold the Reindex
// completion counters of up to kScratchMaxQueries queries at a fixed place:
// zero when the module loads and left at zero by every call, so nothing has
// to clear them (and no memset enters a captured graph).  The rest holds the
// step's workspace, whose layout changes with the call's sizes; no part of
// it needs to start at zero.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kScratchMaxQueries = 65536;
constexpr size_t kScratchCounterBytes = (size_t)kScratchMaxQueries * 4;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The scratch array's device address on the current device, looked up once
// per device (the array's host-side name is not a device address).
static csa2_status scratch_ptr(unsigned char** out) {
  static std::mutex mu;
  static unsigned char* ptrs[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(CSA2_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    ptrs[dev] = (unsigned char*)p;
  }
  *out = ptrs[dev];
  return CSA2_OK;
}

// The layer step's workspace: the Full index's (pool + block scores), then
// the Reindex one (its counters first), then the attention partials.
static size_t step_ws_full(const csa2_dims* d, const csa2_queries* q) { return full_ws(d, q) + pkey_ws(d, q); }
static size_t step_ws_reindex(const csa2_dims* d, const csa2_queries* q) { return align256(reindex_ws(d, q)); }

csa2_status csa2_decode_step_workspace_size(const csa2_dims* d, const csa2_queries* q, size_t* bytes) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (!bytes) return fail(CSA2_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = step_ws_full(d, q) + step_ws_reindex(d, q) + attend_ws(d, q);
  return CSA2_OK;
}

static csa2_status decode_step(const csa2_dims* d, const csa2_queries* q, int32_t mode, const uint8_t* idx_q,
                               const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                               const uint8_t* idx_k_scales, int32_t* pool_blocks, int32_t* pool_count,
                               int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                               float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                               const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base, float* out,
                               float* lse, void* ws, size_t ws_bytes, void* stream, const csa2_pages* pages,
                               uint32_t* counters = nullptr) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (mode != CSA2_LAYER_FULL && mode != CSA2_LAYER_REINDEX && mode != CSA2_LAYER_REUSE)
    return fail(CSA2_ERR_INVALID_ARG, "mode must be CSA2_LAYER_FULL, _REINDEX or _REUSE (got %d)", mode);
  if ((idx_q_scales == nullptr) != (idx_k_scales == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "idx_q_scales and idx_k_scales must both be given (FP4 rows) or both NULL");
  const bool fp4 = idx_q_scales != nullptr;
  // (with external counters the Reindex part holds only its order keys)
  const size_t n_full = step_ws_full(d, q);
  const size_t n_re = counters ? reindex_keys_ws(d, q) : step_ws_reindex(d, q);
  const size_t need = n_full + n_re + attend_ws(d, q);
  if ((st = check_ws(ws, ws_bytes, need))) return st;
  char* w_full = (char*)ws;
  char* w_re = w_full + n_full;
  char* w_att = w_re + n_re;
  const size_t n_att = ws_bytes - n_full - n_re;
  // every stage's arguments are checked before the first launch
  for (int pass = 0; pass < 2; ++pass) {
    const bool dry = pass == 0;
    if (mode == CSA2_LAYER_FULL) {
      // the scan also keeps every position's score; the pool and the Top-K
      // (the layer's own query: what Reindex would compute) are then
      // selected inside the attention kernel
      const size_t n_idx = full_ws(d, q);
      uint32_t* pkey = (uint32_t*)(w_full + n_idx);
      if (!topk_pos || !topk_count) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
      if ((st = index_full(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, fp4, pool_blocks, pool_count,
                           nullptr, 0, w_full, n_idx, stream, dry, pages, pkey, topk_pos, topk_count, true)))
        return st;
      if ((st = pool_topk_attend(d, q, (const float*)(w_full + pool_ws(d, q)), full_ldb(d, q), pkey, full_ldpk(d, q),
                                 pool_blocks, pool_count, topk_pos, topk_count, q_lat, q_rope, softmax_scale,
                                 kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out, lse, w_full, pool_ws(d, q),
                                 CSA2_POOL_WS_FROM_SCAN, attend_ws(d, q) ? w_att : nullptr, n_att, stream, dry,
                                 pages)))
        return st;
      continue;
    }
    if (mode == CSA2_LAYER_REINDEX) {
      // the attention workgroups select the Top-K from the Reindex keys
      if ((st = reindex_attend(d, q, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count,
                               topk_pos, topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope,
                               swa_kv, swa_base, out, lse, w_re, n_re, attend_ws(d, q) ? w_att : nullptr, n_att,
                               stream, dry, counters, pages)))
        return st;
      continue;
    }
    // a Reuse layer: attention on the inherited Top-K
    if ((st = attend(d, q, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv,
                     swa_base, out, lse, attend_ws(d, q) ? w_att : nullptr, n_att, stream, dry, pages)))
      return st;
  }
  return CSA2_OK;
}

csa2_status csa2_decode_step(const csa2_dims* d, const csa2_queries* q, int32_t mode, const uint8_t* idx_q,
                             const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                             const uint8_t* idx_k_scales, int32_t* pool_blocks, int32_t* pool_count,
                             int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                             float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                             const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base, float* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_step(d, q, mode, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count, topk_pos,
                     topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out,
                     lse, ws, ws_bytes, stream, nullptr);
}

csa2_status csa2_decode_step_noalloc(const csa2_dims* d, const csa2_queries* q, int32_t mode, const uint8_t* idx_q,
                                     const uint8_t* idx_q_scales, const float* idx_w, const uint8_t* idx_k,
                                     const uint8_t* idx_k_scales, int32_t* pool_blocks, int32_t* pool_count,
                                     int32_t* topk_pos, int32_t* topk_count, const uint16_t* q_lat,
                                     const uint16_t* q_rope, float softmax_scale, const uint8_t* kv_codes,
                                     const uint8_t* kv_scales, const uint16_t* kv_rope, const uint16_t* swa_kv,
                                     const int64_t* swa_base, float* out, float* lse, void* stream) {
  csa2_status st = check_dims(d);
  if (st) return st;
  if ((st = check_queries(q))) return st;
  if (q->n_q > kScratchMaxQueries)
    return fail(CSA2_ERR_WORKSPACE, "csa2_decode_step_noalloc takes at most %d queries (got %d)", kScratchMaxQueries,
                q->n_q);
  const size_t need = step_ws_full(d, q) + reindex_keys_ws(d, q) + attend_ws(d, q);
  const size_t have = kScratchBytes - kScratchCounterBytes;
  if (need > have)
    return fail(CSA2_ERR_WORKSPACE, "csa2_decode_step_noalloc: this batch needs %zu bytes of scratch, the maximum is %zu",
                need, have);
  if ((st = check_device())) return st;
  unsigned char* base = nullptr;
  if ((st = scratch_ptr(&base))) return st;
  return decode_step(d, q, mode, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count, topk_pos,
                     topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out,
                     lse, base + kScratchCounterBytes, have, stream, nullptr, (uint32_t*)base);
}

csa2_status csa2_decode_step_paged(const csa2_dims* d, const csa2_queries* q, const csa2_pages* pages,
                                   int32_t mode, const uint8_t* idx_q, const uint8_t* idx_q_scales,
                                   const float* idx_w, const uint8_t* idx_k, const uint8_t* idx_k_scales,
                                   int32_t* pool_blocks, int32_t* pool_count, int32_t* topk_pos,
                                   int32_t* topk_count, const uint16_t* q_lat, const uint16_t* q_rope,
                                   float softmax_scale, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                   const uint16_t* kv_rope, const uint16_t* swa_kv, const int64_t* swa_base,
                                   float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!pages) return fail(CSA2_ERR_INVALID_ARG, "pages is NULL");
  return decode_step(d, q, mode, idx_q, idx_q_scales, idx_w, idx_k, idx_k_scales, pool_blocks, pool_count, topk_pos,
                     topk_count, q_lat, q_rope, softmax_scale, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, out,
                     lse, ws, ws_bytes, stream, pages);
}

csa2_status csa2_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || (bytes & 15)) return fail(CSA2_ERR_INVALID_ARG, "bytes must be a non-negative multiple of 16");
  if (bytes > 0 && (!buf || !sink)) return fail(CSA2_ERR_INVALID_ARG, "required pointer is NULL");
  if (((uintptr_t)buf & 15) || ((uintptr_t)sink & 3)) return fail(CSA2_ERR_INVALID_ARG, "misaligned buffer");
  csa2_status st = check_device();
  if (st) return st;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = launch_stream_read(buf, bytes, sink, g_cus[dev], (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "stream read launch");
}

}  // extern "C"
