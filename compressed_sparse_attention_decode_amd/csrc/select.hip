// Top-P block pool selection (Full mode, second half).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (hierarchical sparse indexer: the
// Full layer keeps the Top-2048 blocks of 8 as the candidate pool).  Order is
// (block score descending, block id ascending); the pool is written in
// ascending block order.
//
// Keys are order-preserving uint32 images of the block scores.  A batch
// whose queries all have at most kPoolSmallBlocks (16,384) blocks is selected
// by k_pool_small, one workgroup per query (see the end of this file).
// Otherwise, since one CU streams a few tens of GB/s at most, a long context
// (131,056 blocks at 1M) is split into chunks of 4096 blocks, each handled by
// its own workgroup:
//  K1 k_pool_minmax: per chunk, the smallest and largest key; chunk 0 also
//     clears the query's global histogram.  (The Full scan can write these
//     (min, max) pairs per scan tile and clear the histogram itself; then K1
//     is skipped.)
//  K2 k_pool_hist: a histogram over 4096 linear bins of the query's score
//     range [min, max] (monotone in the key, and spread evenly; bit digits of
//     scores that share an exponent would pile onto a few counters); per
//     chunk in LDS, then added to the query's histogram.
//  K3 k_pool_mark: every chunk finds the bin b* holding the P-th best block,
//     writes its blocks of higher bins as a bitmap and lists its blocks of
//     bin b* as candidates.  The last chunk workgroup of the query to finish
//     then runs the final step: the candidates (usually a few dozen) are
//     ranked exactly against each other by (key desc, block asc) and the
//     best join the selection (more than 128 candidates: an exact radix
//     select over the bits below their common prefix gives the threshold key
//     and how many blocks equal to it are needed, admitted lowest id first);
//     the ordered compaction of the bitmap writes ascending block ids; the
//     histogram is cleared again.  If a chunk listed more candidates than
//     its slots, this step re-reads the block scores instead (correct for
//     any input, slow only for near-constant scores).
#include <mutex>

#include "common.h"
#include "internal.h"
#include "radix_topk.h"
#include "pool_topk.h"
#include "select_common.h"
#include "topk_positions.h"

namespace csa2 {
namespace {

constexpr int kCT = 1024;                      // chunk workgroup threads
constexpr int kCU = kPoolChunk / (kCT * 4);    // 16-byte block-score loads per chunk thread
constexpr int kCandCap = 2048;                 // candidates the final step holds in LDS
constexpr int kRankCap = 128;                 // candidates ranked exactly against each other (quadratic)
static_assert(kPoolChunk == kCT * 4 * kCU, "a chunk thread holds 4 kCU blocks");

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// keys agree on every bit >= lo (lo in [0, 32])
__device__ __forceinline__ bool same_above(uint32_t a, uint32_t b, int lo) {
  return ((uint64_t)a >> lo) == ((uint64_t)b >> lo);
}

struct PoolWs {
  uint32_t* hist;     // [kHistBins]
  uint32_t* mm;       // [mm_cap][2] min, max key per span of blocks
  uint32_t* cnt;      // [G] candidates listed per chunk (may exceed the slots)
  uint32_t* done;     // [1] chunk workgroups of K3 finished (K2 clears it)
  uint32_t* sel;      // [G * kPoolChunk / 32] bitmap of blocks above bin b*
  uint32_t* ckey;     // [G][kPoolChunkCand]
  int32_t* cblk;      // [G][kPoolChunkCand]
};

__device__ __forceinline__ PoolWs pool_ws(const PoolArgs& a, int q) {
  PoolWs w;
  const int G = a.chunks;
  w.hist = a.ws + (int64_t)q * a.ws_stride;
  w.mm = w.hist + kHistBins;
  w.cnt = w.mm + 2 * a.mm_cap;
  w.done = w.cnt + G;
  w.sel = w.done + 1;
  w.ckey = w.sel + G * (kPoolChunk / 32);
  w.cblk = reinterpret_cast<int32_t*>(w.ckey + G * kPoolChunkCand);
  return w;
}

__device__ __forceinline__ int query_blocks(const PoolArgs& a, int q) {
  const int c = max(0, a.n_visible[q] - a.swa);
  return (c + 7) >> 3;
}

// The thread's 4 kCU blocks of a chunk: kCU 16-byte loads, block e of load u
// is jb0(u) + e with jb0(u) = base + (u * kCT + tid) * 4.  The loads are bounded
// by the row stride only (a multiple of 4 floats), so they need not wait for
// the query's block count; blocks >= nb are masked afterwards.
struct ChunkKeys {
  v4f x[kCU];
  uint32_t k[kCU][4];
  uint32_t vm[kCU];
  __device__ __forceinline__ void load(const float* bs, int base, int64_t ld, int tid) {
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int jb0 = base + (u * kCT + tid) * 4;
      x[u] = jb0 < ld ? *reinterpret_cast<const v4f*>(bs + jb0) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  __device__ __forceinline__ void finish(int base, int nb, int tid) {
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int left = nb - (base + (u * kCT + tid) * 4);
      vm[u] = left >= 4 ? 15u : (left <= 0 ? 0u : (1u << left) - 1u);
#pragma unroll
      for (int e = 0; e < 4; ++e) k[u][e] = order_key(x[u][e]);
    }
  }
};

// The query's key range from the (min, max) pairs of its spans of blocks
// (chunks of K1, or scan tiles).  load() issues the thread's first kKrPer
// pairs (clamped to the workspace, so before the block count is known);
// reduce() masks them by the count and reads any further pairs.
constexpr int kKrPer = 4;
template <int NT>
struct KeyRange {
  v2u m[kKrPer];
  __device__ __forceinline__ void load(const PoolArgs& a, const PoolWs& w) {
#pragma unroll
    for (int r = 0; r < kKrPer; ++r)
      m[r] = *reinterpret_cast<const v2u*>(w.mm + 2 * min((int)threadIdx.x + r * NT, a.mm_cap - 1));
  }
  __device__ __forceinline__ void reduce(const PoolArgs& a, const PoolWs& w, int nb, uint32_t* s_scan,
                                         uint32_t* kmin, uint32_t* kmax) {
    const int nb1 = a.mm_half * a.mm_span1;
    const int n = min(a.mm_cap, nb <= nb1 ? (nb + a.mm_span1 - 1) / a.mm_span1
                                          : a.mm_half + (nb - nb1 + a.mm_span - 1) / a.mm_span);
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int r = 0; r < kKrPer; ++r) {
      const bool v = (int)threadIdx.x + r * NT < n;
      lo = min(lo, v ? m[r][0] : 0xFFFFFFFFu);
      hi = max(hi, v ? m[r][1] : 0u);
    }
    for (int i = threadIdx.x + kKrPer * NT; i < n; i += NT) {
      const v2u x = *reinterpret_cast<const v2u*>(w.mm + 2 * i);
      lo = min(lo, x[0]);
      hi = max(hi, x[1]);
    }
    block_minmax_u32<NT>(&lo, &hi, s_scan);
    *kmin = lo;
    *kmax = hi;
  }
};

// kHistBins linear bins of the score range [min, max]: monotone in the key
// (so bins order the keys) and, unlike bit digits of scores that share an
// exponent, spread evenly.  All keys equal (or a range that overflows): one bin.
struct Bins {
  float lo, scale;
  __device__ __forceinline__ uint32_t bin(uint32_t key) const {
    return (uint32_t)min((int)((key_float(key) - lo) * scale), kHistBins - 1);
  }
};

__device__ __forceinline__ Bins bins_for(uint32_t kmin, uint32_t kmax) {
  Bins b;
  b.lo = key_float(kmin);
  b.scale = (float)kHistBins / (key_float(kmax) - b.lo);
  if (!(b.scale > 0.0f && b.scale < 3.0e38f)) b.scale = 0.0f;
  return b;
}

// The thread's histogram bins, counted from the top: bin kHistBins-1-(tid*kPer+k).
template <int NT>
struct HistSlice {
  static constexpr int kPer = kHistBins / NT;
  uint32_t c[kPer];
  __device__ __forceinline__ void load(const uint32_t* hist) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kPer; k += 4) {
      const v4u x = *reinterpret_cast<const v4u*>(hist + kHistBins - (tid + 1) * kPer + k);
      c[kPer - 1 - k] = x[0]; c[kPer - 2 - k] = x[1]; c[kPer - 3 - k] = x[2]; c[kPer - 4 - k] = x[3];
    }
  }
};

// Bin b* of the P-th best key and the number of keys in higher bins:
// s_out[0] = b*, s_out[1] = above.
template <int NT>
__device__ __forceinline__ void find_bstar(const HistSlice<NT>& h, uint32_t P, uint32_t* s_scan, uint32_t* s_out) {
  constexpr int kPer = HistSlice<NT>::kPer;
  const int tid = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) local += h.c[k];
  uint32_t total;
  uint32_t above = block_exclusive_scan<NT>(local, s_scan, &total);
  if (above < P && P <= above + local) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (above < P && P <= above + h.c[k]) {
        s_out[0] = kHistBins - 1 - (tid * kPer + k);
        s_out[1] = above;
      }
      above += h.c[k];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- K1
__global__ __launch_bounds__(kCT) void k_pool_minmax(PoolArgs a) {
  __shared__ uint32_t s_scan[2 * (kCT / 64)];
  const int q = blockIdx.x / a.chunks, g = blockIdx.x % a.chunks, tid = threadIdx.x;
  const PoolWs w = pool_ws(a, q);
  if (g == 0) {
    for (int i = tid * 4; i < kHistBins; i += kCT * 4)
      *reinterpret_cast<v4u*>(w.hist + i) = v4u{0u, 0u, 0u, 0u};
  }
  const int base = g * kPoolChunk;
  ChunkKeys c;
  c.load(a.bscore + (int64_t)q * a.ld, base, a.ld, tid);
  const int nb = query_blocks(a, q);
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  if (nb > a.pool && base < nb) {
    c.finish(base, nb, tid);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c.vm[u] >> e & 1u) {
          lo = min(lo, c.k[u][e]);
          hi = max(hi, c.k[u][e]);
        }
      }
    }
  }
  block_minmax_u32<kCT>(&lo, &hi, s_scan);
  if (tid == 0) {
    w.mm[2 * g] = lo;
    w.mm[2 * g + 1] = hi;
  }
}

// ---------------------------------------------------------------- K2
// A workgroup histograms a run of its query's chunks (one chunk, unless
// that grid would exceed two workgroups per CU; the runs are the marking
// kernel's) into LDS, then adds the nonzero bins to the query's histogram.
__global__ __launch_bounds__(kCT) void k_pool_hist(PoolArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_scan[2 * (kCT / 64)];
  const int WPQ = a.mark_wgs;
  const int q = blockIdx.x / WPQ, wq = blockIdx.x % WPQ, tid = threadIdx.x;
  const int cpw = (a.chunks + WPQ - 1) / WPQ;
  const int g0 = wq * cpw, g1 = min(a.chunks, g0 + cpw);
  const PoolWs w = pool_ws(a, q);
  const float* bsq = a.bscore + (int64_t)q * a.ld;
  ChunkKeys c;
  c.load(bsq, g0 * kPoolChunk, a.ld, tid);
  KeyRange<kCT> kr;
  kr.load(a, w);
  if (wq == 0 && tid == 0) *w.done = 0;
  const int nb = query_blocks(a, q);
  if (nb <= a.pool || g0 >= g1 || g0 * kPoolChunk >= nb) return;
  for (int i = tid; i < kHistBins; i += kCT) s_hist[i] = 0;
  uint32_t kmin, kmax;
  kr.reduce(a, w, nb, s_scan, &kmin, &kmax);     // its barriers order the clear
  const Bins b = bins_for(kmin, kmax);
  for (int g = g0; g < g1 && g * kPoolChunk < nb; ++g) {
    const int base = g * kPoolChunk;
    if (g != g0) c.load(bsq, base, a.ld, tid);
    c.finish(base, nb, tid);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c.vm[u] >> e & 1u) atomicAdd(&s_hist[b.bin(c.k[u][e])], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < kHistBins; i += kCT) {
    const uint32_t h = s_hist[i];
    if (h) atomicAdd(&w.hist[i], h);
  }
}

// ---------------------------------------------------------------- K3 + K4
// What a marking workgroup already knows of its query (the same for every
// chunk): the key range, the bin b* and the count of blocks above it.
struct MarkState {
  bool valid;
  uint32_t kmin, kmax, bstar, above;
};

// The final step of one query, run by the last of its chunk workgroups
// (NT threads).  dyn: LDS of 2 * nw_cap + 2 * kCandCap words (the selection
// and tie bitmaps, the gathered candidates).  With a valid MarkState the
// histogram and the key-range pairs are not read again.
template <int NT>
__device__ __forceinline__ void pool_final(const PoolArgs& a, int q, const PoolWs& w, uint32_t* dyn,
                                           const MarkState& ms) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_off[kMaxBlocks / kPoolChunk + 1];
  __shared__ uint32_t s_scan[2 * (NT / 64)];
  __shared__ uint32_t s_misc[4];
  uint32_t* s_sel = dyn;
  uint32_t* s_tie = dyn + a.nw_cap;
  uint32_t* s_ckey = dyn + 2 * a.nw_cap;
  int32_t* s_cj = reinterpret_cast<int32_t*>(s_ckey + kCandCap);

  const int tid = threadIdx.x;
  const int P = a.pool, G = a.chunks;
  const float* bs = a.bscore + (int64_t)q * a.ld;
  const int nb = query_blocks(a, q);
  int32_t* out = a.pool_blocks + (int64_t)q * P;
  if (nb <= P) {
    for (int j = tid; j < P; j += NT) out[j] = j < nb ? j : -1;
    if (tid == 0) a.pool_count[q] = nb;
    for (int i = tid * 4; i < kHistBins; i += NT * 4) *reinterpret_cast<v4u*>(w.hist + i) = v4u{0u, 0u, 0u, 0u};
    return;
  }
  const int nw = (nb + 31) >> 5;

  // every independent read issued before the first wait: the bitmap of
  // blocks above b*, the histogram, the chunks' candidate counts, the
  // key-range pairs
  constexpr int kSelPer = (kMaxBlocks / 32 + NT - 1) / NT;
  uint32_t selw[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) selw[k] = w.sel[min(tid + k * NT, nw - 1)];
  const uint32_t cnt_v = w.cnt[min(tid, G - 1)];
  uint32_t kmin = ms.kmin, kmax = ms.kmax, bstar = ms.bstar, above = ms.above;
  if (!ms.valid) {                       // uniform: the workgroup marked no chunk
    HistSlice<NT> h;
    h.load(w.hist);
    KeyRange<NT> kr;
    kr.load(a, w);
    kr.reduce(a, w, nb, s_scan, &kmin, &kmax);
    find_bstar<NT>(h, (uint32_t)P, s_scan, s_misc);
    bstar = s_misc[0];
    above = s_misc[1];
  }
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = tid + k * NT;
    if (i < nw) { s_sel[i] = selw[k]; s_tie[i] = 0; }
  }
  const Bins b = bins_for(kmin, kmax);
  uint32_t need = (uint32_t)P - above;

  // candidate lists of the chunks (offsets by a wave-0 scan over <= 64 chunks)
  if (tid < 64) {
    const uint32_t v = tid < G ? cnt_v : 0u;
    const bool over = v > (uint32_t)kPoolChunkCand;
    const uint32_t x = wave_incl_scan_u32(v);
    if (tid < G) s_off[tid] = x - v;
    const uint64_t ov = __ballot(over);
    if (tid == 63) {
      s_off[G] = x;
      s_misc[2] = (ov != 0 || x > (uint32_t)kCandCap) ? 1u : 0u;   // fall back to the block scores
    }
  }
  __syncthreads();
  const uint32_t C = s_off[G];
  const bool in_lds = s_misc[2] == 0;
  if (in_lds) {
    const int wave = tid >> 6, lane = tid & 63;
    for (int g = wave; g < G; g += NT / 64) {
      const uint32_t n = s_off[g + 1] - s_off[g];
      for (uint32_t i = lane; i < n; i += 64) {
        s_ckey[s_off[g] + i] = w.ckey[(int64_t)g * kPoolChunkCand + i];
        s_cj[s_off[g] + i] = w.cblk[(int64_t)g * kPoolChunkCand + i];
      }
    }
  }
  __syncthreads();

  // Up to kRankCap candidates held in LDS are ranked exactly against each
  // other by (key desc, block asc); the best `need` join the selection.
  // Otherwise a radix select over the candidates' own key range finds the
  // threshold key T and how many blocks equal to T are needed, admitted
  // lowest block first.
  const bool ranked = in_lds && C <= (uint32_t)kRankCap;
  uint32_t need_eq = 0;
  if (ranked) {
    for (uint32_t i = tid; i < C; i += NT) {
      const uint32_t ki = s_ckey[i];
      const int ji = s_cj[i];
      uint32_t r = 0;
#pragma unroll 8
      for (uint32_t j = 0; j < C; ++j) {
        const uint32_t kj = s_ckey[j];
        r += kj > ki || (kj == ki && s_cj[j] < ji);
      }
      if (r < need) atomicOr(&s_sel[ji >> 5], 1u << (ji & 31));
    }
    __syncthreads();
  } else {
    // the candidates' own key range: its common leading bits are decided
    uint32_t clo = 0xFFFFFFFFu, chi = 0;
    if (in_lds) {
      for (uint32_t i = tid; i < C; i += NT) { clo = min(clo, s_ckey[i]); chi = max(chi, s_ckey[i]); }
    } else {
      for (int jb = tid; jb < nb; jb += NT) {
        const uint32_t key = order_key(bs[jb]);
        if (b.bin(key) == bstar) { clo = min(clo, key); chi = max(chi, key); }
      }
    }
    block_minmax_u32<NT>(&clo, &chi, s_scan);
    int fixed_lo = highest_diff_bit(clo, chi) + 1;     // bits >= fixed_lo are decided
    uint32_t prefix = (uint32_t)(((uint64_t)clo >> fixed_lo) << fixed_lo);
    while (fixed_lo > 0) {
      const int sh = max(0, fixed_lo - 8);
      const uint32_t dmask = (1u << (fixed_lo - sh)) - 1;
      for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t i = tid; i < C; i += NT) {
          const uint32_t key = s_ckey[i];
          if (same_above(key, prefix, fixed_lo)) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
        }
      } else {
        for (int jb = tid; jb < nb; jb += NT) {
          const uint32_t key = order_key(bs[jb]);
          if (b.bin(key) == bstar && same_above(key, prefix, fixed_lo))
            atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
        }
      }
      __syncthreads();
      find_crossing(s_hist, 256, need, s_misc);
      __syncthreads();
      prefix |= s_misc[0] << sh;
      need -= s_misc[1];
      fixed_lo = sh;
      __syncthreads();
    }
    const uint32_t T = prefix;
    need_eq = need;
    // candidates above T join the selection; those equal to T are tie bits
    if (in_lds) {
      for (uint32_t i = tid; i < C; i += NT) {
        const uint32_t key = s_ckey[i];
        const int jb = s_cj[i];
        if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
        else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
      }
    } else {
      for (int jb = tid; jb < nb; jb += NT) {
        const uint32_t key = order_key(bs[jb]);
        if (b.bin(key) != bstar) continue;
        if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
        else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
      }
    }
    __syncthreads();
  }

  // ordered compaction (ties, in the radix path, admitted in ascending block order)
  const int wpt = (nw + NT - 1) / NT;
  const int w_lo = min(nw, tid * wpt), w_hi = min(nw, w_lo + wpt);
  uint32_t total;
  if (!ranked) {
    uint32_t ties = 0;
    for (int i = w_lo; i < w_hi; ++i) ties += __popc(s_tie[i]);
    uint32_t tie_before = block_exclusive_scan<NT>(ties, s_scan, &total);
    for (int i = w_lo; i < w_hi; ++i) {
      uint32_t t = s_tie[i], acc = 0;
      while (t && tie_before < need_eq) {
        const uint32_t bit = t & (0u - t);
        acc |= bit;
        t ^= bit;
        ++tie_before;
      }
      s_sel[i] |= acc;
    }
  }
  uint32_t sel_local = 0;
  for (int i = w_lo; i < w_hi; ++i) sel_local += __popc(s_sel[i]);
  uint32_t out_before = block_exclusive_scan<NT>(sel_local, s_scan, &total);
  for (int i = w_lo; i < w_hi; ++i) {
    uint32_t fin = s_sel[i];
    while (fin) {
      const int bit = __ffs(fin) - 1;
      fin &= fin - 1;
      if (out_before < (uint32_t)P) out[out_before] = i * 32 + bit;
      ++out_before;
    }
  }
  if (tid == 0) a.pool_count[q] = P;
  // leave the histogram cleared: a later pool call on the same scan-prepared
  // workspace (the same block scores) accumulates onto zero again
  for (int i = tid * 4; i < kHistBins; i += NT * 4) *reinterpret_cast<v4u*>(w.hist + i) = v4u{0u, 0u, 0u, 0u};
}

// Marking per chunk; the last marking workgroup of a query to finish
// (counted in the workspace's done word, which K2 clears) runs the final
// step.  A workgroup marks a run of its query's chunks (one chunk, unless the
// grid would exceed two workgroups per CU: then fewer workgroups take several
// chunks each, and the key range and the bin b* are found once per
// workgroup).  The marks cross workgroups through memory: after a store
// drain and a barrier, one release fence per workgroup publishes them before
// it counts itself in, and the last one's acquire fence makes the others'
// visible.
__global__ __launch_bounds__(kCT) void k_pool_mark(PoolArgs a) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_scan[2 * (kCT / 64)];
  __shared__ uint32_t s_misc[2];
  __shared__ uint32_t s_ccount;
  __shared__ uint32_t s_last;
  const int WPQ = a.mark_wgs;
  const int q = blockIdx.x / WPQ, wq = blockIdx.x % WPQ;
  const int cpw = (a.chunks + WPQ - 1) / WPQ;
  const int g0 = wq * cpw, g1 = min(a.chunks, g0 + cpw);
  const int tid = threadIdx.x, lane = tid & 63;
  const PoolWs w = pool_ws(a, q);
  const float* bsq = a.bscore + (int64_t)q * a.ld;
  ChunkKeys c;
  c.load(bsq, g0 * kPoolChunk, a.ld, tid);     // the first chunk's scores, before the rest
  HistSlice<kCT> h;
  h.load(w.hist);
  KeyRange<kCT> kr;
  kr.load(a, w);
  const int nb = query_blocks(a, q);
  MarkState ms = {false, 0u, 0u, 0u, 0u};
  const bool marks = nb > a.pool && g0 < g1 && g0 * kPoolChunk < nb;   // uniform
  Bins b{};
  uint32_t bstar = 0;
  if (marks) {
    uint32_t kmin, kmax;
    kr.reduce(a, w, nb, s_scan, &kmin, &kmax);
    b = bins_for(kmin, kmax);
    find_bstar<kCT>(h, (uint32_t)a.pool, s_scan, s_misc);
    bstar = s_misc[0];
    ms = {true, kmin, kmax, bstar, s_misc[1]};
  }
  for (int g = g0; g < g1; ++g) {
    const int base = g * kPoolChunk;
    if (!(marks && base < nb)) {
      if (tid == 0) w.cnt[g] = 0;
      continue;
    }
    if (g != g0) c.load(bsq, base, a.ld, tid);
    c.finish(base, nb, tid);
    if (tid == 0) s_ccount = 0;
    __syncthreads();                        // the count is cleared (and the last chunk's read)

    uint32_t* ck = w.ckey + (int64_t)g * kPoolChunkCand;
    int32_t* cj = w.cblk + (int64_t)g * kPoolChunkCand;
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int jb0 = base + (u * kCT + tid) * 4;
      uint32_t hib = 0, cand = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v = c.vm[u] >> e & 1u;
        const uint32_t bin = b.bin(c.k[u][e]);
        hib |= (uint32_t)(v && bin > bstar) << e;
        cand |= (uint32_t)(v && bin == bstar) << e;
      }
      // a lane's 4 blocks form one nibble; 8 lanes OR their nibbles into a word
      uint32_t word = hib << (4 * (lane & 7));
      word |= __shfl_xor(word, 1, 64);
      word |= __shfl_xor(word, 2, 64);
      word |= __shfl_xor(word, 4, 64);
      if ((lane & 7) == 0 && jb0 < nb) w.sel[jb0 >> 5] = word;
      uint64_t m[4];
      uint32_t tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = __ballot(cand >> e & 1u);
        tot += (uint32_t)__popcll(m[e]);
      }
      if (tot == 0) continue;                       // wave-uniform
      uint32_t slot0 = 0;
      if (lane == 0) slot0 = atomicAdd(&s_ccount, tot);
      slot0 = __shfl(slot0, 0, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cand >> e & 1u) {
          const uint32_t slot = slot0 + lane_prefix(m[e]);
          if (slot < (uint32_t)kPoolChunkCand) { ck[slot] = c.k[u][e]; cj[slot] = jb0 + e; }
        }
        slot0 += (uint32_t)__popcll(m[e]);
      }
    }
    __syncthreads();
    if (tid == 0) w.cnt[g] = s_ccount;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores have reached L2
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t prev = __hip_atomic_fetch_add(w.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(WPQ - 1);
    if (s_last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      *w.done = 0;
    }
  }
  __syncthreads();
  if (!s_last) return;
  pool_final<kCT>(a, q, w, s_dyn, ms);
}

// ---------------------------------------------------------------- small pools
// A query with at most kPoolSmallBlocks blocks (contexts up to 131,200
// positions) is selected by one 512-thread workgroup (pool_topk.h): one
// launch instead of the histogram and marking kernels, with the same
// result.  With BPT > 0 the same workgroup then takes the Full layer's
// Top-K from the scan's position keys.
static_assert(kPoolSmallBlocks == kMaxCand, "one key per register slot");

template <int BPT>
__global__ __launch_bounds__(kTkThreads) void k_pool_small(PoolArgs a) {
  __shared__ PoolTopkLds<BPT> s_sel;
  const int q = blockIdx.x;
  PoolTopkOut o;
  o.pool = a.pool_blocks + (int64_t)q * a.pool;
  o.pool_count = a.pool_count + q;
  o.topk = BPT > 0 ? a.topk_pos + (int64_t)q * a.topk : nullptr;
  o.topk_count = BPT > 0 ? a.topk_count + q : nullptr;
  o.rows = nullptr;
  o.r0 = o.r1 = 0;
  pool_topk_select<BPT>(a.bscore + (int64_t)q * a.ld, (int)a.ld, query_blocks(a, q), a.pool, a.topk,
                        BPT > 0 ? a.pkey + (int64_t)q * a.ld_pkey : nullptr, o, s_sel, [] {});
}

}  // namespace

// After the chunked selection's words: the scan's group keys (one per
// kGroupBlocks blocks, for the in-kernel selections of long queries).
int64_t pool_gkey_off(int chunks, int mm_cap) {
  const int64_t words = kHistBins + 2 * (int64_t)mm_cap + chunks + 1 + (int64_t)chunks * (kPoolChunk / 32) +
                        2 * (int64_t)chunks * kPoolChunkCand;
  return (words + 3) / 4 * 4;
}

int64_t pool_ws_words(int chunks, int mm_cap) {
  const int64_t words = pool_gkey_off(chunks, mm_cap) + (int64_t)chunks * (kPoolChunk / kGroupBlocks);
  return (words + 63) / 64 * 64;
}

size_t pool_final_lds(int nw_cap) { return ((size_t)2 * nw_cap + 2 * kCandCap) * 4; }

hipError_t launch_pool_select(const PoolArgs& a, hipStream_t s) {
  if (a.small) {
    const dim3 grid((unsigned)a.n_q), block(kTkThreads);
    // twice K's blocks where K allows: room for the crossing bin's extra
    // candidates (K <= 2048 = kTkThreads * 4 in any case)
    if (!a.topk_pos) hipLaunchKernelGGL(k_pool_small<0>, grid, block, 0, s, a);
    else if (a.topk <= kTkThreads) hipLaunchKernelGGL(k_pool_small<2>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k_pool_small<4>, grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (a.topk_pos) return hipErrorInvalidValue;   // the chunked path leaves the Top-K to k_topk_keys
  const dim3 grid((unsigned)(a.n_q * a.chunks));
  const dim3 mgrid((unsigned)(a.n_q * a.mark_wgs));
  const size_t lds = pool_final_lds(a.nw_cap);
  // dynamic LDS above the default limit must be allowed, once per device for
  // the largest size asked so far (the record is per device and locked, so
  // calls on several threads and devices agree)
  if (lds > 48 * 1024) {
    static std::mutex mu;
    static size_t lds_allowed[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (lds > lds_allowed[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pool_mark),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      lds_allowed[dev] = lds;
    }
  }
  if (!a.have_minmax) hipLaunchKernelGGL(k_pool_minmax, grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(k_pool_hist, mgrid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(k_pool_mark, mgrid, dim3(kCT), lds, s, a);
  return hipGetLastError();
}

}  // namespace csa2
