// Core attention over the kept FP4 entries and the bf16 sliding window, with
// one softmax and a 512-wide latent output per head (MLA-absorbed).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (heterogeneous KV: the same main Q
// attends the sparse main-KV branch and the uncompressed window branch and
// the two are merged; mode table: Reuse layers change only Q) and §4 of the
// newsaint.id page (FP4 main KV dequantised just before attention).  The key
// of a sparse entry is [dequantised latent (512) || bf16 rope (64)] and its
// value is the dequantised latent; a window row supplies both from bf16.
// The FP4 scales cover 16 channels, or 32 in the group-32 codec variant (the
// akhunji.com page, "Microscopic FP4 (E2M1) Cache Compression"): a 16-channel
// item then reads the scale byte of its 32-channel group.
//
// Mapping (gfx950): a workgroup = 8 waves = one query x 32 heads x one split
// of the query's tile list.  Waves 0-3 serve heads 0-15 of the 32, waves 4-7
// heads 16-31; within a group, wave w (quarter w & 3) takes entries
// 16w .. 16w+15 of each tile in Q.K^T and output dims 128w .. 128w+127 in
// P.V, so the 64-entry tile image and the query are read once per head group
// instead of once per wave.  The window's positions [c, n) come first (tiles
// of 64 window rows, known before any index arrives), then the kept entries
// (tiles of 64 of topk_pos); a tile never mixes the two.
//  * gathers go straight from HBM into LDS (buffer loads with the LDS
//    destination, 16 bytes per lane), with the wait counts kept by hand: a
//    kept-entry tile's codes, scales and rope are loaded two tiles ahead into
//    one of two staging slots, so two tiles' gathers are in flight while one
//    is contracted; a window tile's rows land directly in the image (its
//    rope in a staging slot), the first one before the loop;
//  * the image is f16 (FP4 x E4M3 values are exact in f16, bf16 window values
//    are exact inside the f16 normal range, the reason for |x| < 65504):
//    kept entries are dequantised from their staging slot, window rows are
//    converted in place;
//  * Q.K^T: v_mfma_f32_16x16x32_f16 over the 512 latent dims with 16 entries
//    of the image as A and the wave's 16 query heads as B (held in
//    registers), and v_mfma_f32_16x16x32_bf16 over the 64 rope dims straight
//    from the staged bf16 rope (the query's rope stays bf16: exact);
//  * online softmax in the exp2 domain: the tile maximum per head is shared
//    through LDS by the group's four waves, P is rounded to f16 (bf16 would
//    cost about 2^-9 relative per weight) and written to LDS as [head][entry];
//  * P.V: v_mfma_f32_16x16x32_f16 with P from LDS as A and the image's values
//    read with the gfx950 transpose read (ds_read_b64_tr_b16) as B, into 8
//    accumulator tiles (16 heads x 128 dims) per wave;
//  * the result goes through LDS so that every output row (512 floats of one
//    head) is written with whole 16-byte stores;
//  * with several splits per (query, head group), each split writes its
//    unnormalised partial (o, m, l) per head and k_attend_combine merges them
//    with a log-sum-exp rescale.  The splits are sized so that the grid fills
//    the chip about once: for a decode batch of a few queries each split is
//    one tile, so a query's work is spread over tens of CUs.
#include "common.h"
#include "internal.h"
#include "group_topk.h"
#include "pool_topk.h"

namespace csa2 {
namespace {

constexpr int kTE = kAttendTile;              // 64 entries per tile
constexpr int kNW = kAttendWaves;             // 8 waves
constexpr int kNT = 64 * kNW;                 // 512 threads
constexpr int kLS = kLatent + 8;              // f16 row stride of the latent image
constexpr int kPS = kTE + 4;                  // f16 row stride of the P tile (rows on distinct banks)
constexpr int kOS = kLatent + 4;              // f32 row stride of the output rows in LDS (a lane group's
                                              // rows 4 gq + i then fall on distinct banks)
constexpr int kMaxRows = kAttendMaxTiles * kTE;          // rows of one split, at most
constexpr int kRowPer = kMaxRows / kNT;                  // rows resolved per thread
constexpr int kItems = kTE * 64 / kNT;        // (entry, 8-channel half group) items per thread
constexpr int kWinRow = kKeyDim * 2;          // bytes of a window row
constexpr uint32_t kOob = 0xFFFFFF00u;        // a buffer offset past any row: reads zero
constexpr int32_t kNoRow = 0x7FFFFFFF;

// LDS layout (bytes): the latent image, two rope slots, two staging slots
// (codes, then the tile's scale block), the split's row codes, P, and the
// per-head maxima, rescales and sums.  At the end the output rows reuse the
// image and rope slots.
constexpr int kOffLat = 0;
constexpr int kOffRope = kOffLat + kTE * kLS * 2;
constexpr int kRopeSlot = kTE * kRope * 2;
constexpr int kOffStage = kOffRope + 2 * kRopeSlot;
constexpr int kCodeStage = kTE * kCodeBytes;
constexpr int kStageSlot = kCodeStage + kNW * 256;
constexpr int kOffRow = kOffStage + 2 * kStageSlot;
constexpr int kOffP = kOffRow + kMaxRows * 4;
constexpr int kOffMx = kOffP + 2 * 16 * kPS * 2;
constexpr int kOffAl = kOffMx + 2 * 4 * 16 * 4;
constexpr int kOffLw = kOffAl + 2 * 16 * 4;
constexpr int kLdsBytes = kOffLw + 2 * 4 * 16 * 4;
// A selecting split's query latents (32 rows of 512 bf16, padded so that the
// 16 rows one read instruction spans fall on distinct banks), in the image
// after the selection's own LDS; read into registers before the first gather.
constexpr int kQS = (kLatent + 8) * 2;
constexpr int kOffQ = 18 * 1024;
static_assert(kOffQ + kAttendHeads * kQS <= kTE * kLS * 2, "query latents fit in the image");
// a selecting split's candidate groups (long queries), in the image after the
// query latents
constexpr int kOffGrp = kOffQ + kAttendHeads * kQS;
constexpr int kOffGrpBits = kOffGrp + 4 * 4 * kTkThreads;   // their bitmap
static_assert(kOffGrp % 16 == 0 && kOffGrpBits + 4 * kMaxGroups / 32 <= kTE * kLS * 2,
              "candidate groups and their bitmap fit in the image");
static_assert(kOffGrp + 4 * kMaxCand <= kOffRow, "a Reindex selection's staged keys fit before the row codes");
static_assert(sizeof(PoolGroupLds) <= kLdsBytes, "a pool selection fits the workgroup's LDS");
static_assert(kMaxGroups == kPoolGroupsMax, "the host's bound of the group keys");
static_assert(kTE * 8 == kNT, "one rope chunk per thread");
static_assert(kRowPer % 2 == 0, "rows resolved per thread in two halves");
static_assert(kTE * kScaleBytes <= kNW * 256, "a tile's scale block: one 256-byte load per wave");
static_assert(kAttendHeads * kOS * 4 <= kOffStage, "output rows fit in the image and rope slots");
static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));

// bf16 pair -> f16 pair.  Exact for values inside the f16 range (the ABI's
// |x| < 65504 precondition); round-toward-zero only matters outside it.
__device__ __forceinline__ uint32_t bf16x2_to_h2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)));
}

// Four code bytes (eight E2M1 values, low nibble first) times an E4M3 scale,
// as four f16 pairs.  The gfx950 conversion at scale 1.0 is exact, and so is
// the f16 product: E2M1 x E4M3 needs at most 6 significant bits and lies in
// [2^-13, 2688].
template <int B>
__device__ __forceinline__ uint32_t fp4_byte_h2(uint32_t word, v2h s2) {
  const v2h x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, B);
  return __builtin_bit_cast(uint32_t, x * s2);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// Buffer resource (as four SGPRs) over [base, base + bytes): loads past the
// end return zeros.
__device__ __forceinline__ v4u rsrc_of(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return v4u{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) & 0xFFFFu,
             (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// Buffer loads with the LDS as destination: lane l's 16 (or 4) bytes land at
// the wave-uniform LDS address `lds` + 16 l (+ 4 l).  They count in vmcnt like
// any load; the compiler does not see them, so every wait for them is written
// out (wait_vmcnt below).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t off, v4u rsrc) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t off, v4u rsrc) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc) : "memory", "m0");
}

// s_waitcnt vmcnt(N) (gfx9 layout: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]; the fields not named are left at "no wait").  Loads retire
// in order, so vmcnt(N) means: all but the N youngest loads have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// The loads issued ahead for one tile, per wave: a kept-entry tile 4 (two
// code loads, one scale load, one rope load), a window tile 1 (its rope).
constexpr int kAheadSparse = 4;
constexpr int kAheadWindow = 1;
__device__ __forceinline__ void wait_ahead(int n) {
  if (n == kAheadSparse) wait_vmcnt<kAheadSparse>();
  else if (n == kAheadWindow) wait_vmcnt<kAheadWindow>();
  else wait_vmcnt<0>();
}

// Maximum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_rows4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// SEL > 0: the splits with kept-entry tiles select the query's Full-layer
// Top-K themselves (pool_topk.h, SEL blocks per thread in its positions
// step) instead of reading topk_pos: the selection is repeated by each such
// split, which costs a few microseconds of one CU each, against a launch and
// a round trip for the positions; the split holding the first kept-entry
// tile of head group 0 writes the Top-K out.  SRC: where the selection
// starts.  kSrcScan: the scan's block scores and position keys; one extra
// workgroup per query (past the attention grid) selects and writes the pool,
// so the attention splits need only the Top-K's candidate blocks (those at
// or above the first histogram's bound for the K-th block); kSrcPool: the
// pool is given (a query too long for one workgroup's selection), the splits
// select only its Top-K; kSrcReindex: a Reindex layer's Top-K from the order
// keys its scoring kernel wrote (csa2_reindex_attend); kSrcGroups: as
// kSrcScan, and a query longer than one workgroup's registers hold
// (kMaxCand blocks) selects from the scan's group keys (group_topk.h).
constexpr int kSrcScan = 0, kSrcPool = 1, kSrcReindex = 2, kSrcGroups = 3;
// PGD (SEL > 0): paged main-KV planes; the selected positions become rows
// through the page table before the gathers.  (SEL == 0 reads a.pages.)
template <int SEL, int SRC, bool PGD = false>
__global__ __launch_bounds__(kNT) void k_attend(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[kLdsBytes];
  _Float16* s_lat = reinterpret_cast<_Float16*>(s_mem + kOffLat);   // [64][kLS]
  int32_t* s_row = reinterpret_cast<int32_t*>(s_mem + kOffRow);     // [kMaxRows]
  _Float16* s_p = reinterpret_cast<_Float16*>(s_mem + kOffP);       // [2 groups][16 heads * kPS]
  float* s_mx = reinterpret_cast<float*>(s_mem + kOffMx);           // [2][4 quarters][16]: tile maximum per head
  float* s_al = reinterpret_cast<float*>(s_mem + kOffAl);           // [2][16]: this tile's rescale per head
  float* s_lw = reinterpret_cast<float*>(s_mem + kOffLw);           // [2][4][16]: row sums per head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, col = lane & 15;
  const int hgl = wave >> 2, qw = wave & 3;       // head group (of 16) in the workgroup, quarter
  const int S = a.splits, HG = a.head_groups;
  if constexpr (SEL > 0 && (SRC == kSrcScan || SRC == kSrcGroups)) {
    // one workgroup per query past the attention grid selects and writes the
    // pool (the attention workgroups then need only the Top-K's candidates)
    const int main_grid = a.n_q * HG * S;
    if ((int)blockIdx.x >= main_grid) {
      const int qp = (int)blockIdx.x - main_grid;
      const int cp = max(0, load_uniform(a.n_visible + qp) - a.swa);
      PoolTopkOut o;
      o.pool = a.pool_blocks + (int64_t)qp * a.pool;
      o.pool_count = a.pool_count + qp;
      o.topk = nullptr;
      o.topk_count = nullptr;
      o.rows = nullptr;
      o.r0 = o.r1 = 0;
      const int nbq = (cp + 7) >> 3;
      if (SRC == kSrcGroups && nbq > kMaxCand)
        pool_from_groups(a.gkey + (int64_t)qp * a.ld_gkey, a.gcap, a.bscore + (int64_t)qp * a.ld_bs, a.ld_bs, nbq,
                         a.pool, o.pool, o.pool_count, *reinterpret_cast<PoolGroupLds*>(s_mem));
      else
        pool_topk_select<0>(a.bscore + (int64_t)qp * a.ld_bs, (int)a.ld_bs, nbq, a.pool, a.topk, nullptr, o,
                            *reinterpret_cast<PoolTopkLds<0>*>(s_mem + kOffLat), [] {});
      return;
    }
  }
  const int q = blockIdx.x / (HG * S);
  const int hg = (blockIdx.x / S) % HG;
  const int sp = blockIdx.x % S;
  const int H = a.heads, K = a.topk;
  const int head0 = hg * kAttendHeads + hgl * 16;  // the wave's 16 heads: head0 .. head0 + 15
  const int nwt = (a.swa + kTE - 1) / kTE;        // window tiles (of the plan: W rows)
  const int t_begin = sp * a.split_tiles;
  const int t_end = min(nwt + (K + kTE - 1) / kTE, t_begin + a.split_tiles);
  const int ntl = max(0, t_end - t_begin);
  // the query's sizes and bases: scalar loads issued together, one round
  // trip (a use between them would wait for the first alone)
  const int n = load_uniform(a.n_visible + q);
  const int tcount = SEL ? 0 : load_uniform(a.topk_count + q);
  const int pcount = SRC != kSrcScan ? load_uniform(a.pool_count + q) : 0;
  const int64_t sbase = load_uniform(a.seq_base + q);
  const int64_t wbase = load_uniform(a.swa_base + q);

  // the split's kept positions (the row always holds K entries), then the
  // wave's 16 query heads: both in flight together
  int32_t tkv[kRowPer];
  if constexpr (SEL == 0) {
    const int32_t* tk = a.topk_pos + (int64_t)q * K;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const int idx = tid + j * kNT;
      const int jj = (t_begin + idx / kTE - nwt) * kTE + idx % kTE;   // index in topk_pos (sparse tiles)
      tkv[j] = tk[min(max(jj, 0), K - 1)];
    }
  }
  // lane (col, gq) holds head head0 + col, dims 32 ks + 8 gq .. + 8 (a
  // selecting split issues these after its block-score loads)
  v4u rq[kKeyDim / 32];
  auto load_q = [&]() {
    const int64_t qh = (int64_t)q * H + min(head0 + col, H - 1);
#pragma unroll
    for (int ks = 0; ks < kKeyDim / 32; ++ks) {
      const int d = ks * 32 + gq * 8;
      rq[ks] = *reinterpret_cast<const v4u*>(d < kLatent ? a.q_lat + qh * kLatent + d : a.q_rope + qh * kRope + (d - kLatent));
    }
  };
  const bool selects = SEL > 0 && t_end > nwt;
  if (!selects) load_q();
  // a selecting split: the latent dims into the LDS (one 1 KiB row per
  // instruction instead of every wave loading its group's 16 heads), the
  // rope dims into registers, both issued once the block keys are in
  auto load_q_sel = [&]() {
    const v4u rs_q = rsrc_of(a.q_lat + (int64_t)q * H * kLatent, (uint32_t)H * (kLatent * 2));
#pragma unroll
    for (int j = 0; j < kAttendHeads / kNW; ++j) {
      const int h = (kAttendHeads / kNW) * wave + j;
      dma16(lds_addr(s_mem + kOffQ + h * kQS), (uint32_t)min(hg * kAttendHeads + h, H - 1) * (kLatent * 2) + lane * 16,
            rs_q);
    }
    const int64_t qh = (int64_t)q * H + min(head0 + col, H - 1);
#pragma unroll
    for (int j = 0; j < kRope / 32; ++j)
      rq[kLatent / 32 + j] = *reinterpret_cast<const v4u*>(a.q_rope + qh * kRope + j * 32 + gq * 8);
  };
  const int c = max(0, n - a.swa);
  const int Ew = n - c;                           // window rows [c, n)
  int Es = min(tcount, K);
  // paged main KV: the kept positions become rows of the whole planes (one
  // page id per position, loaded unconditionally from a clamped slot)
  const bool paged = SEL == 0 ? a.pages != nullptr : PGD;
  if (SEL == 0 && paged && c > 0) {
    int32_t pg[kRowPer];
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) pg[j] = a.pages[sbase + (min(max(tkv[j], 0), c - 1) >> a.page_shift)];
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) asm volatile("" : "+v"(pg[j]));
#pragma unroll
    for (int j = 0; j < kRowPer; ++j)
      tkv[j] = (int32_t)(((uint32_t)pg[j] << a.page_shift) | ((uint32_t)tkv[j] & ((1u << a.page_shift) - 1u)));
  }
  // the query's sources, each over exactly its rows
  const int64_t kbase = paged ? 0 : sbase;
  const uint32_t krows = paged ? (uint32_t)a.rows : (uint32_t)n;
  const int gshift = a.kv_gshift;
  const uint32_t sbytes = (uint32_t)kScaleBytes >> gshift;
  const v4u rs_codes = rsrc_of(a.kv_codes + kbase * kCodeBytes, krows * kCodeBytes);
  const v4u rs_scales = rsrc_of(a.kv_scales + kbase * sbytes, krows * sbytes);
  const v4u rs_rope = rsrc_of(a.kv_rope + kbase * kRope, krows * (kRope * 2));
  const v4u rs_win = rsrc_of(a.swa_kv + wbase * kKeyDim, (uint32_t)Ew * kWinRow);
  // row codes of the split's tiles (>= 0: cache row, < 0: window row -1 - code)
  asm volatile("" ::"s"(n), "s"(tcount), "s"(pcount), "s"(sbase), "s"(wbase));
#pragma unroll
  for (int j = 0; j < kRowPer; ++j) {
    const int idx = tid + j * kNT;
    if (idx < ntl * kTE) {
      const int t = t_begin + idx / kTE, e = idx % kTE;
      int32_t code = kNoRow;
      if (t < nwt) {
        const int ge = t * kTE + e;
        if (ge < Ew) code = -1 - ge;
      } else if (SEL == 0 && (t - nwt) * kTE + e < Es) {
        code = tkv[j];
      }
      s_row[idx] = code;
    }
  }
  if constexpr (SEL > 0) {
    if (selects) {
      // this split's kept positions (ranks r0 .. r1 of the Top-K) straight
      // into its row codes; the selection's LDS is the image's, unused until
      // the first gather (its first barrier orders the row codes above)
      static_assert(sizeof(PoolTopkLds<SEL>) <= kOffQ, "selection LDS fits in the image before the query");
      const int s_first = max(t_begin, nwt);
      const bool lead = hg == 0 && t_begin <= nwt;  // holds the first kept-entry tile
      PoolTopkOut o;
      o.pool = nullptr;                           // (written by the pool workgroups, or given)
      o.pool_count = nullptr;
      o.topk = lead ? a.topk_out + (int64_t)q * K : nullptr;
      o.topk_count = lead ? a.topk_count_out + q : nullptr;
      o.rows = s_row + (s_first - t_begin) * kTE;
      o.r0 = (s_first - nwt) * kTE;
      o.r1 = (t_end - nwt) * kTE;
      PoolTopkLds<SEL>& sl = *reinterpret_cast<PoolTopkLds<SEL>*>(s_mem + kOffLat);
      uint32_t kept;
      if constexpr (SRC == kSrcReindex)
        kept = topk_from_keys(a.rkeys + (int64_t)q * a.pool * kBlock, a.pool_blocks + (int64_t)q * a.pool,
                              min(pcount, a.pool), a.pool, K, o, sl.radix, sl.scan,
                              reinterpret_cast<uint32_t*>(s_mem + kOffGrp), load_q_sel);
      else if constexpr (SRC == kSrcPool)
        kept = topk_from_pool<SEL>(a.pool_blocks + (int64_t)q * a.pool, min(pcount, a.pool), a.pool,
                                   a.bscore + (int64_t)q * a.ld_bs, a.pkey + (int64_t)q * a.ld_pkey, K, o, nullptr,
                                   sl, load_q_sel);
      else if (SRC == kSrcGroups && ((c + 7) >> 3) > a.group_min)
        kept = topk_from_groups<SEL>(a.gkey + (int64_t)q * a.ld_gkey, a.gcap, a.bscore + (int64_t)q * a.ld_bs, a.ld_bs,
                                     (c + 7) >> 3, a.pkey + (int64_t)q * a.ld_pkey, K, o, sl,
                                     reinterpret_cast<int32_t*>(s_mem + kOffGrp),
                                     reinterpret_cast<uint32_t*>(s_mem + kOffGrpBits), load_q_sel);
      else if (K <= a.pool)                       // (the K best blocks lie in the pool)
        kept = topk_from_blocks<SEL>(a.bscore + (int64_t)q * a.ld_bs, (int)a.ld_bs, (c + 7) >> 3,
                                     a.pkey + (int64_t)q * a.ld_pkey, K, o, sl,
                                     reinterpret_cast<uint32_t*>(s_mem + kOffGrp), load_q_sel);
      else
        kept = pool_topk_select<SEL>(a.bscore + (int64_t)q * a.ld_bs, (int)a.ld_bs, (c + 7) >> 3, a.pool, K,
                                     a.pkey + (int64_t)q * a.ld_pkey, o, sl, load_q_sel);
      Es = min((int)kept, K);
      if (PGD && c > 0) {
        // paged main KV: this split's kept positions (written by the
        // selection, whose last barrier made them visible) become rows of
        // the whole planes, one page id each; a half of the thread's rows at
        // a time with its loads issued together (the second half only for
        // splits of more than 3 kNT rows: fewer live registers)
        constexpr int kHalf = kRowPer / 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && ntl * kTE <= kHalf * kNT) break;
          int32_t pos[kHalf], pg[kHalf];
#pragma unroll
          for (int j = 0; j < kHalf; ++j) {
            const int idx = tid + (h * kHalf + j) * kNT;
            pos[j] = idx < ntl * kTE ? s_row[idx] : kNoRow;
            pg[j] = a.pages[sbase + (min(max(pos[j], 0), c - 1) >> a.page_shift)];
          }
#pragma unroll
          for (int j = 0; j < kHalf; ++j) {
            const int idx = tid + (h * kHalf + j) * kNT;
            if (pos[j] >= 0 && pos[j] != kNoRow)
              s_row[idx] = (int32_t)(((uint32_t)pg[j] << a.page_shift) | ((uint32_t)pos[j] & ((1u << a.page_shift) - 1u)));
          }
        }
      }
      wait_vmcnt<0>();                             // this wave's query rows have landed
    }
  }
  __syncthreads();
  if (selects) {
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ++ks)
      rq[ks] = *reinterpret_cast<const v4u*>(s_mem + kOffQ + (hgl * 16 + col) * kQS + (ks * 32 + gq * 8) * 2);
    __syncthreads();                              // read before any gather lands in the image
  }
  auto tile_entries = [&](int t) {
    return t < nwt ? min(kTE, max(0, Ew - t * kTE)) : min(kTE, max(0, Es - (t - nwt) * kTE));
  };

  // ---- gathers.  Rope: rows 8 wave .. +8, lane l -> row 8 wave + l / 8 and
  // source chunk (l % 8) ^ (l / 8), so a row's chunk j sits at position
  // j ^ (row % 8) and the Q.K^T reads of 8 rows fall on distinct banks.
  auto issue_rope = [&](int ti, bool win) {
    const int32_t* rows = s_row + ti * kTE;
    const int ne = tile_entries(t_begin + ti);
    const int r = 8 * wave + (lane >> 3);
    const int32_t code = rows[r];
    const uint32_t ch = (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
    const uint32_t dst = lds_addr(s_mem + kOffRope + (ti & 1) * kRopeSlot + 8 * wave * (kRope * 2));
    if (win) dma16(dst, r < ne ? (uint32_t)(-1 - code) * kWinRow + kLatent * 2 + ch : kOob, rs_win);
    else dma16(dst, r < ne ? (uint32_t)code * (kRope * 2) + ch : kOob, rs_rope);
  };
  // a kept-entry tile: codes (rows 8 wave .. +8, two KiB loads of 4 rows),
  // the wave's 256 bytes of the tile's scale block, the rope
  auto issue_sparse = [&](int ti) {
    const int32_t* rows = s_row + ti * kTE;
    const int ne = tile_entries(t_begin + ti);
    unsigned char* st = s_mem + kOffStage + (ti & 1) * kStageSlot;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * wave + 4 * h + (lane >> 4);
      dma16(lds_addr(st + (8 * wave + 4 * h) * kCodeBytes),
            r < ne ? (uint32_t)rows[r] * kCodeBytes + (lane & 15) * 16 : kOob, rs_codes);
    }
    const int b = wave * 256 + lane * 4;          // byte of the [64][sbytes] scale block
    const int r = b >> (5 - gshift);
    dma4(lds_addr(st + kCodeStage + wave * 256),
         r < ne ? (uint32_t)rows[min(r, kTE - 1)] * sbytes + ((uint32_t)b & (sbytes - 1)) : kOob, rs_scales);
    issue_rope(ti, false);
  };
  // a window tile's latent rows, straight into the image (bf16 for now)
  auto issue_window_rows = [&](int ti) {
    const int32_t* rows = s_row + ti * kTE;
    const int ne = tile_entries(t_begin + ti);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 8 * wave + j;
      const int32_t code = rows[r];
      dma16(lds_addr(s_lat + r * kLS), r < ne ? (uint32_t)(-1 - code) * kWinRow + lane * 16 : kOob, rs_win);
    }
  };
  auto is_window = [&](int ti) { return t_begin + ti < nwt; };
  auto ahead_count = [&](int ti) { return ti >= ntl ? 0 : (is_window(ti) ? kAheadWindow : kAheadSparse); };
  auto issue_ahead = [&](int ti) {
    if (ti >= ntl) return;
    if (is_window(ti)) issue_rope(ti, true);
    else issue_sparse(ti);
  };

  if (ntl > 0) {
    issue_ahead(0);
    if (is_window(0)) issue_window_rows(0);
  }
  issue_ahead(1);

  // the query as MFMA operands: latent dims in f16, rope dims in bf16 (the
  // empty asm keeps the wait for the query loads here, after the gathers are
  // issued)
#pragma unroll
  for (int ks = 0; ks < kKeyDim / 32; ++ks) asm volatile("" : "+v"(rq[ks]));
  v8h qf[kLatent / 32];
  v8bf qr[kRope / 32];
  {
    const bool live = head0 + col < H;
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ++ks) {
      const v4u x = live ? rq[ks] : v4u{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(v8h, (v4u{bf16x2_to_h2(x[0]), bf16x2_to_h2(x[1]), bf16x2_to_h2(x[2]), bf16x2_to_h2(x[3])}));
    }
#pragma unroll
    for (int j = 0; j < kRope / 32; ++j)
      qr[j] = __builtin_bit_cast(v8bf, live ? rq[kLatent / 32 + j] : v4u{0u, 0u, 0u, 0u});
  }

  float m = -__builtin_inff(), l = 0.0f;         // per head (lanes of column col), this lane's entries' sum
  v4f o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ti = 0; ti < ntl; ++ti) {
    const int t = t_begin + ti;
    const int ne = tile_entries(t);
    const bool win = t < nwt;
    const unsigned char* rope = s_mem + kOffRope + (ti & 1) * kRopeSlot;
    if (win && ti > 0) {
      __syncthreads();                            // the previous tile's reads of the image are done
      issue_window_rows(ti);
      wait_vmcnt<0>();
    } else {
      wait_ahead(ahead_count(ti + 1));            // this tile's loads have landed (the next tile's in flight)
    }
    __syncthreads();                              // every wave's loads have landed; the previous P.V is done
    if (ne > 0) {
      if (win) {
        // window rows in place: bf16 -> f16
#pragma unroll
        for (int j = 0; j < kTE * (kLatent / 8) / kNT; ++j) {
          const int idx = j * kNT + tid, r = idx >> 6, ch = idx & 63;
          v4u* p = reinterpret_cast<v4u*>(s_lat + r * kLS + ch * 8);
          const v4u x = *p;
          *p = v4u{bf16x2_to_h2(x[0]), bf16x2_to_h2(x[1]), bf16x2_to_h2(x[2]), bf16x2_to_h2(x[3])};
        }
      } else {
        // kept entries: codes x scale from the staging slot (a lane writes
        // 16 consecutive bytes of the image, so a wave's writes are whole rows)
        const unsigned char* st = s_mem + kOffStage + (ti & 1) * kStageSlot;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
          const int it = tid + k * kNT, e = it >> 6, hg8 = it & 63;
          const uint32_t cw = *reinterpret_cast<const uint32_t*>(st + e * kCodeBytes + hg8 * 4);
          // the E4M3 scale by the hardware conversion (OCP E4M3FN, exact;
          // 0x7F / 0xFF are NaN as the format defines them)
          const _Float16 sh =
              (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)st[kCodeStage + e * sbytes + ((hg8 >> 1) >> gshift)], 0);
          const v2h s2 = {sh, sh};
          *reinterpret_cast<v4u*>(s_lat + e * kLS + hg8 * 8) =
              v4u{fp4_byte_h2<0>(cw, s2), fp4_byte_h2<1>(cw, s2), fp4_byte_h2<2>(cw, s2), fp4_byte_h2<3>(cw, s2)};
        }
      }
    }
    __syncthreads();                              // the image is complete

    // ---- S^T = K . Q^T for entries 16 qw .. +16 (two accumulator chains)
    float sv[4];
    if (ne > 0) {
      v4f s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
      const int er = 16 * qw + col;
      const _Float16* kr = s_lat + er * kLS + gq * 8;
      // eight K fragments in flight: each read's LDS latency hides behind
      // the MFMAs of the seven before it
      constexpr int kKF = 8;
      v4u kf[kKF];
#pragma unroll
      for (int j = 0; j < kKF; ++j) kf[j] = *reinterpret_cast<const v4u*>(kr + j * 32);
#pragma unroll
      for (int ks = 0; ks < kLatent / 32; ++ks) {
        const v8h k = __builtin_bit_cast(v8h, kf[ks % kKF]);
        if (ks + kKF < kLatent / 32) kf[ks % kKF] = *reinterpret_cast<const v4u*>(kr + (ks + kKF) * 32);
        if (ks & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qf[ks], s1, 0, 0, 0);
        else s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qf[ks], s0, 0, 0, 0);
      }
      // keep that order: the scheduler otherwise trades the reads in flight
      // for registers and waits out every read's latency
      __builtin_amdgcn_sched_group_barrier(0x100, kKF, 0);
#pragma unroll
      for (int j = 0; j < kLatent / 32 - kKF; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kKF, 0);
      {
        const unsigned char* rr = rope + er * (kRope * 2);
        const v8bf r0 = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(rr + ((gq ^ (er & 7)) * 16)));
        const v8bf r1 = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(rr + (((4 + gq) ^ (er & 7)) * 16)));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, qr[0], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1, qr[1], s1, 0, 0, 0);
      }
      // lane holds entries 16 qw + 4 gq + i for head col
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = 16 * qw + 4 * gq + i < ne ? (s0[i] + s1[i]) * a.scale_log2 : -__builtin_inff();
      const float wmax = max_rows4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      if (gq == 0) s_mx[(hgl * 4 + qw) * 16 + col] = wmax;
    }
    __syncthreads();                              // maxima written; every wave is past its Q.K^T
    issue_ahead(ti + 2);                          // into the slots this tile has finished with
    if (ne == 0) continue;

    const float* mx = s_mx + hgl * 64;
    const float tmax = fmaxf(fmaxf(mx[col], mx[16 + col]), fmaxf(mx[32 + col], mx[48 + col]));
    const float m_new = fmaxf(m, tmax);           // finite: the tile has an entry
    const float alpha = exp2f(m - m_new);
    float ps = 0.0f;
    _Float16 ph[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sv[i] - m_new);
      ps += p;
      ph[i] = (_Float16)p;
    }
    l = l * alpha + ps;
    m = m_new;
    _Float16* pg = s_p + hgl * 16 * kPS;
    *reinterpret_cast<v4s*>(&pg[col * kPS + 16 * qw + 4 * gq]) = __builtin_bit_cast(v4s, (v4h_t{ph[0], ph[1], ph[2], ph[3]}));
    if (qw == 0 && gq == 0) s_al[hgl * 16 + col] = alpha;
    __syncthreads();

    // ---- O[heads][dims 128 qw ..] = alpha O + P . V
    const v4f ar = *reinterpret_cast<const v4f*>(&s_al[hgl * 16 + 4 * gq]);    // alpha of heads 4 gq + i
    const bool same = ar[0] == 1.0f && ar[1] == 1.0f && ar[2] == 1.0f && ar[3] == 1.0f;
    if (__builtin_amdgcn_ballot_w64(!same) != 0) {      // (uniform) some head's maximum moved
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= ar[i];
      }
    }
    const int ra_ = 4 * gq + (col >> 2), cb = 4 * (col & 3);
#pragma unroll
    for (int kk = 0; kk < kTE / 32; ++kk) {
      // k-slots: entries 32 kk + 4 gq .. +4, then 32 kk + 16 + 4 gq .. +4 (the
      // transpose read hands lane col the same entries of dim 16 nt + col)
      const v2u plo = *reinterpret_cast<const v2u*>(&pg[col * kPS + 32 * kk + 4 * gq]);
      const v2u phi = *reinterpret_cast<const v2u*>(&pg[col * kPS + 32 * kk + 16 + 4 * gq]);
      const v8h pa = __builtin_bit_cast(v8h, (v4u{plo[0], plo[1], phi[0], phi[1]}));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int d = 128 * qw + nt * 16 + cb;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s_lat + (32 * kk + ra_) * kLS + d));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s_lat + (32 * kk + 16 + ra_) * kLS + d));
        const v8h vb = __builtin_bit_cast(v8h, (v4u{__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1],
                                                    __builtin_bit_cast(v2u, hi)[0], __builtin_bit_cast(v2u, hi)[1]}));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[nt], 0, 0, 0);
      }
    }
  }

  // ---- row sums per head: this lane's entries, the four lane groups, the
  // group's four waves
  const float lw = sum_rows4(l);
  if (gq == 0) s_lw[(hgl * 4 + qw) * 16 + col] = lw;
  __syncthreads();                                // also: every wave is past its last P.V
  const float* lwg = s_lw + hgl * 64;
  const float l_head = (lwg[col] + lwg[16 + col]) + (lwg[32 + col] + lwg[48 + col]);
  // lane holds O[head 4 gq + i][dim 128 qw + 16 nt + col]
  float li[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * gq + i;
    li[i] = (lwg[hh] + lwg[16 + hh]) + (lwg[32 + hh] + lwg[48 + hh]);
  }

  // ---- the 32 rows (normalised, or this split's unnormalised partial)
  // through LDS, then whole 16-byte stores
  const bool fin = S == 1;
  float* s_o = reinterpret_cast<float*>(s_mem);  // [32 heads][kOS]
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s_o[(hgl * 16 + 4 * gq + i) * kOS + 128 * qw + nt * 16 + col] =
          fin ? (li[i] > 0.0f ? o[nt][i] / li[i] : 0.0f) : o[nt][i];
  }
  __syncthreads();
  const int HP = HG * kAttendHeads;
  float* dst = fin ? a.out + ((int64_t)q * H + hg * kAttendHeads) * kLatent
                   : a.part_o + (((int64_t)q * S + sp) * HP + hg * kAttendHeads) * kLatent;
#pragma unroll
  for (int j = 0; j < kAttendHeads * (kLatent / 4) / kNT; ++j) {
    const int idx = j * kNT + tid, hr = idx >> 7, c4 = (idx & 127) * 4;
    if (hg * kAttendHeads + hr < H)
      *reinterpret_cast<v4f*>(dst + hr * kLatent + c4) = *reinterpret_cast<const v4f*>(s_o + hr * kOS + c4);
  }
  if (qw == 0 && gq == 0 && head0 + col < H) {
    if (fin) {
      if (a.lse)
        a.lse[(int64_t)q * H + head0 + col] = l_head > 0.0f ? (m + log2f(l_head)) * 0.69314718055994531f : -__builtin_inff();
    } else {
      *reinterpret_cast<v2f*>(a.part_ml + (((int64_t)q * S + sp) * HP + head0 + col) * 2) = v2f{m, l_head};
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// lse = M + log2(sum_s 2^(m_s - M) l_s) (in the exp2 domain, then as a
// natural log).  A thread owns four dims of one head and issues every
// split's loads before the first use: one round trip.
// SM: a bound of the split count (2, 4, 8, 10, 12 or 16), so that only the
// splits that exist are loaded.
constexpr int kCombineThreads = 256;     // two heads x 128 threads of 4 dims
template <int SM>
__global__ __launch_bounds__(kCombineThreads) void k_attend_combine(AttendArgs a) {
  const int S = a.splits, H = a.heads, HP = a.head_groups * kAttendHeads;
  const int q = blockIdx.x / (HP / 2);
  const int h = (blockIdx.x % (HP / 2)) * 2 + (threadIdx.x >> 7);
  const int d = (threadIdx.x & 127) * 4;
  if (h >= H) return;
  v2f ml[SM];
  v4f os[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int64_t r = ((int64_t)q * S + min(s, S - 1)) * HP + h;
    ml[s] = *reinterpret_cast<const v2f*>(a.part_ml + r * 2);
    os[s] = *reinterpret_cast<const v4f*>(a.part_o + r * kLatent + d);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < SM; ++s)
    if (s < S && ml[s][1] > 0.0f) M = fmaxf(M, ml[s][0]);
  float den = 0.0f;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const float w = s < S && ml[s][1] > 0.0f ? exp2f(ml[s][0] - M) : 0.0f;
    den += w * ml[s][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += w * os[s][i];
  }
  v4f r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = den > 0.0f ? acc[i] / den : 0.0f;
  *reinterpret_cast<v4f*>(a.out + ((int64_t)q * H + h) * kLatent + d) = r;
  if (a.lse && d == 0)
    a.lse[(int64_t)q * H + h] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
}

// A selecting attention launch: the paged instance when the planes are paged.
template <int SEL, int SRC>
void launch_sel(const AttendArgs& a, dim3 grid, hipStream_t s) {
  if (a.pages) hipLaunchKernelGGL((k_attend<SEL, SRC, true>), grid, dim3(kNT), 0, s, a);
  else hipLaunchKernelGGL((k_attend<SEL, SRC>), grid, dim3(kNT), 0, s, a);
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.split_tiles * kTE > kMaxRows || a.splits < 1 || a.splits > kAttendMaxSplits ||
      (a.splits > 1 && (!a.part_o || !a.part_ml)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.n_q * a.head_groups * a.splits));
  if (a.rkeys) {
    if (a.pool > 2048 || a.topk > 2048 || !a.pool_blocks || !a.pool_count || !a.topk_out ||
        !a.topk_count_out)
      return hipErrorInvalidValue;
    launch_sel<1, kSrcReindex>(a, grid, s);
  } else if (!a.bscore) {
    hipLaunchKernelGGL((k_attend<0, kSrcScan>), grid, dim3(kNT), 0, s, a);
  } else {
    // (without a given pool: a query of at most kMaxCand blocks, or the
    // group keys; pool and Top-K within 2048: checked by the caller)
    if (a.pool > 2048 || a.topk > 2048 || !a.pkey || !a.pool_blocks || !a.pool_count || !a.topk_out ||
        !a.topk_count_out)
      return hipErrorInvalidValue;
    if (a.sel_from_pool) {
      // (K <= 1024: the positions step of a larger K does not fit the
      // registers beside the attention's; the caller selects it apart)
      if (a.topk <= kTkThreads) launch_sel<1, kSrcPool>(a, grid, s);
      else if (a.topk <= 2 * kTkThreads) launch_sel<2, kSrcPool>(a, grid, s);
      else return hipErrorInvalidValue;
    } else {
      // plus one pool workgroup per query
      const dim3 gp((unsigned)(a.n_q * a.head_groups * a.splits + a.n_q));
      if (a.gkey) {
        // long queries from the group keys: Top-K within 1024 (candidate
        // groups, 512 SEL of them), pool within half the candidate groups
        if (a.topk > 2 * kTkThreads || 2 * a.pool > kPoolGroupCap || a.gcap < 4 || a.gcap % 4 ||
            a.gcap > kMaxGroups || a.ld_gkey < a.gcap || a.group_min < 0 || a.group_min > kMaxCand)
          return hipErrorInvalidValue;
        if (a.topk <= kTkThreads) launch_sel<2, kSrcGroups>(a, gp, s);
        else launch_sel<4, kSrcGroups>(a, gp, s);
      } else if (a.topk <= kTkThreads) {
        launch_sel<2, kSrcScan>(a, gp, s);
      } else {
        launch_sel<4, kSrcScan>(a, gp, s);
      }
    }
  }
  if (a.splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 cg((unsigned)(a.n_q * a.head_groups * kAttendHeads / 2));
    if (a.splits <= 2) hipLaunchKernelGGL(k_attend_combine<2>, cg, dim3(kCombineThreads), 0, s, a);
    else if (a.splits <= 4) hipLaunchKernelGGL(k_attend_combine<4>, cg, dim3(kCombineThreads), 0, s, a);
    else if (a.splits <= 8) hipLaunchKernelGGL(k_attend_combine<8>, cg, dim3(kCombineThreads), 0, s, a);
    else if (a.splits <= 10) hipLaunchKernelGGL(k_attend_combine<10>, cg, dim3(kCombineThreads), 0, s, a);
    else if (a.splits <= 12) hipLaunchKernelGGL(k_attend_combine<12>, cg, dim3(kCombineThreads), 0, s, a);
    else hipLaunchKernelGGL(k_attend_combine<kAttendMaxSplits>, cg, dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace csa2
