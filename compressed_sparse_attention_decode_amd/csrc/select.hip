// Top-P block pool selection (Full mode, second half).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (hierarchical sparse indexer: the
// Full layer keeps the Top-2048 blocks of 8 as the candidate pool).  Order is
// (block score descending, block id ascending); the pool is written in
// ascending block order.
//
// Keys are order-preserving uint32 images of the block scores.  One CU streams
// a few tens of GB/s at most, so a long context (131,056 blocks at 1M) is
// split into chunks of 4096 blocks, each handled by its own workgroup, and
// only the final exact step runs one workgroup per query:
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
//     bin b* as candidates.
//  K4 k_pool_final: the candidates (usually a few dozen) are ranked exactly
//     against each other by (key desc, block asc) and the best join the
//     selection (more than 128 candidates: an exact radix select over the bits
//     below their common prefix gives the threshold key and how many blocks
//     equal to it are needed, admitted lowest id first); the ordered compaction of the
//     bitmap writes ascending block ids; the histogram is cleared again.  If a chunk listed more
//     candidates than its slots, this step re-reads the block scores instead
//     (correct for any input, slow only for near-constant scores).
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace csa2 {
namespace {

constexpr int kCT = 256;                       // chunk workgroup threads
constexpr int kFT = 1024;                      // final workgroup threads
constexpr int kCandCap = 8192;                 // candidates the final step holds in LDS
constexpr int kRankCap = 128;                 // candidates ranked exactly against each other (quadratic)
constexpr int kMaxWords = kMaxBlocks / 32;
static_assert(kPoolChunk == kCT * 16, "a chunk thread holds 16 blocks");
static_assert(kHistBins == 4 * kFT, "the final step clears the histogram 4 words per thread");

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
  w.sel = w.cnt + G;
  w.ckey = w.sel + G * (kPoolChunk / 32);
  w.cblk = reinterpret_cast<int32_t*>(w.ckey + G * kPoolChunkCand);
  return w;
}

__device__ __forceinline__ int query_blocks(const PoolArgs& a, int q) {
  const int c = max(0, a.n_visible[q] - a.swa);
  return (c + 7) >> 3;
}

// The thread's 16 blocks of a chunk: 4 x 16-byte loads, block e of load u is
// jb0(u) + e with jb0(u) = base + (u * kCT + tid) * 4.  The loads are bounded
// by the row stride only (a multiple of 4 floats), so they need not wait for
// the query's block count; blocks >= nb are masked afterwards.
struct ChunkKeys {
  v4f x[4];
  uint32_t k[4][4];
  uint32_t vm[4];
  __device__ __forceinline__ void load(const float* bs, int base, int64_t ld, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jb0 = base + (u * kCT + tid) * 4;
      x[u] = jb0 < ld ? *reinterpret_cast<const v4f*>(bs + jb0) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  __device__ __forceinline__ void finish(int base, int nb, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int left = nb - (base + (u * kCT + tid) * 4);
      vm[u] = left >= 4 ? 15u : (left <= 0 ? 0u : (1u << left) - 1u);
#pragma unroll
      for (int e = 0; e < 4; ++e) k[u][e] = order_key(x[u][e]);
    }
  }
};

// The query's key range from the (min, max) pairs of its spans of blocks
// (chunks of K1, or scan tiles).  load() issues the thread's first pair before
// the block count is known; reduce() masks it and reads any further pairs.
template <int NT>
struct KeyRange {
  v2u m0;
  __device__ __forceinline__ void load(const PoolArgs& a, const PoolWs& w) {
    const int i = threadIdx.x;
    m0 = i < a.mm_cap ? *reinterpret_cast<const v2u*>(w.mm + 2 * i) : v2u{0xFFFFFFFFu, 0u};
  }
  __device__ __forceinline__ void reduce(const PoolArgs& a, const PoolWs& w, int nb, uint32_t* s_scan,
                                         uint32_t* kmin, uint32_t* kmax) {
    const int n = (nb + a.mm_span - 1) / a.mm_span;
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
    if ((int)threadIdx.x < n) { lo = m0[0]; hi = m0[1]; }
    for (int i = threadIdx.x + NT; i < n; i += NT) {
      const v2u m = *reinterpret_cast<const v2u*>(w.mm + 2 * i);
      lo = min(lo, m[0]);
      hi = max(hi, m[1]);
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
    for (int u = 0; u < 4; ++u) {
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
__global__ __launch_bounds__(kCT) void k_pool_hist(PoolArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_scan[2 * (kCT / 64)];
  const int q = blockIdx.x / a.chunks, g = blockIdx.x % a.chunks, tid = threadIdx.x;
  const int base = g * kPoolChunk;
  const PoolWs w = pool_ws(a, q);
  ChunkKeys c;
  c.load(a.bscore + (int64_t)q * a.ld, base, a.ld, tid);
  KeyRange<kCT> kr;
  kr.load(a, w);
  const int nb = query_blocks(a, q);
  if (nb <= a.pool || base >= nb) return;
  c.finish(base, nb, tid);
  for (int i = tid; i < kHistBins; i += kCT) s_hist[i] = 0;
  uint32_t kmin, kmax;
  kr.reduce(a, w, nb, s_scan, &kmin, &kmax);     // its barriers order the clear
  const Bins b = bins_for(kmin, kmax);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c.vm[u] >> e & 1u) atomicAdd(&s_hist[b.bin(c.k[u][e])], 1u);
  }
  __syncthreads();
  for (int i = tid; i < kHistBins; i += kCT) {
    const uint32_t h = s_hist[i];
    if (h) atomicAdd(&w.hist[i], h);
  }
}

// ---------------------------------------------------------------- K3
__global__ __launch_bounds__(kCT) void k_pool_mark(PoolArgs a) {
  __shared__ uint32_t s_scan[2 * (kCT / 64)];
  __shared__ uint32_t s_misc[2];
  __shared__ uint32_t s_ccount;
  const int q = blockIdx.x / a.chunks, g = blockIdx.x % a.chunks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int base = g * kPoolChunk;
  const PoolWs w = pool_ws(a, q);
  ChunkKeys c;
  c.load(a.bscore + (int64_t)q * a.ld, base, a.ld, tid);
  HistSlice<kCT> h;
  h.load(w.hist);
  KeyRange<kCT> kr;
  kr.load(a, w);
  const int nb = query_blocks(a, q);
  if (nb <= a.pool || base >= nb) {
    if (tid == 0) w.cnt[g] = 0;
    return;
  }
  c.finish(base, nb, tid);
  if (tid == 0) s_ccount = 0;
  uint32_t kmin, kmax;
  kr.reduce(a, w, nb, s_scan, &kmin, &kmax);
  const Bins b = bins_for(kmin, kmax);
  find_bstar<kCT>(h, (uint32_t)a.pool, s_scan, s_misc);
  const uint32_t bstar = s_misc[0];

  uint32_t* ck = w.ckey + (int64_t)g * kPoolChunkCand;
  int32_t* cj = w.cblk + (int64_t)g * kPoolChunkCand;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
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

// ---------------------------------------------------------------- K4
__global__ __launch_bounds__(kFT) void k_pool_final(PoolArgs a) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_sel[kMaxWords];
  __shared__ uint32_t s_tie[kMaxWords];
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int32_t s_cj[kCandCap];
  __shared__ uint32_t s_off[kMaxBlocks / kPoolChunk + 1];
  __shared__ uint32_t s_scan[2 * (kFT / 64)];
  __shared__ uint32_t s_misc[4];

  const int q = blockIdx.x, tid = threadIdx.x;
  const int P = a.pool, G = a.chunks;
  const PoolWs w = pool_ws(a, q);
  const float* bs = a.bscore + (int64_t)q * a.ld;

  // every independent read issued before the first wait (none waits for the
  // block count): the bitmap of blocks above b* (the query's whole region),
  // the histogram, the chunks' candidate counts, the key-range pairs
  constexpr int kSelPer = kMaxWords / kFT;
  uint32_t selw[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = tid + k * kFT;
    selw[k] = i < G * (kPoolChunk / 32) ? w.sel[i] : 0u;
  }
  HistSlice<kFT> h;
  h.load(w.hist);
  const uint32_t cnt_v = tid < G ? w.cnt[tid] : 0u;
  KeyRange<kFT> kr;
  kr.load(a, w);
  const int nb = query_blocks(a, q);
  int32_t* out = a.pool_blocks + (int64_t)q * P;
  if (nb <= P) {
    for (int j = tid; j < P; j += kFT) out[j] = j < nb ? j : -1;
    if (tid == 0) a.pool_count[q] = nb;
    return;
  }
  const int nw = (nb + 31) >> 5;
  uint32_t kmin, kmax;
  kr.reduce(a, w, nb, s_scan, &kmin, &kmax);
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = tid + k * kFT;
    if (i < nw) { s_sel[i] = selw[k]; s_tie[i] = 0; }
  }
  const Bins b = bins_for(kmin, kmax);
  find_bstar<kFT>(h, (uint32_t)P, s_scan, s_misc);
  const uint32_t bstar = s_misc[0];
  uint32_t need = (uint32_t)P - s_misc[1];

  // candidate lists of the chunks (offsets by a wave-0 scan over <= 64 chunks)
  if (tid < 64) {
    const uint32_t v = cnt_v;
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
    for (int g = wave; g < G; g += kFT / 64) {
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
  // Otherwise a radix select over bits [0, cs) finds the threshold key T and
  // how many blocks equal to T are needed, admitted lowest block first.
  const bool ranked = in_lds && C <= (uint32_t)kRankCap;
  uint32_t need_eq = 0;
  if (ranked) {
    for (uint32_t i = tid; i < C; i += kFT) {
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
      for (uint32_t i = tid; i < C; i += kFT) { clo = min(clo, s_ckey[i]); chi = max(chi, s_ckey[i]); }
    } else {
      for (int jb = tid; jb < nb; jb += kFT) {
        const uint32_t key = order_key(bs[jb]);
        if (b.bin(key) == bstar) { clo = min(clo, key); chi = max(chi, key); }
      }
    }
    block_minmax_u32<kFT>(&clo, &chi, s_scan);
    int fixed_lo = highest_diff_bit(clo, chi) + 1;     // bits >= fixed_lo are decided
    uint32_t prefix = (uint32_t)(((uint64_t)clo >> fixed_lo) << fixed_lo);
    while (fixed_lo > 0) {
      const int sh = max(0, fixed_lo - 8);
      const uint32_t dmask = (1u << (fixed_lo - sh)) - 1;
      if (tid < 256) s_hist[tid] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t i = tid; i < C; i += kFT) {
          const uint32_t key = s_ckey[i];
          if (same_above(key, prefix, fixed_lo)) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
        }
      } else {
        for (int jb = tid; jb < nb; jb += kFT) {
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
      for (uint32_t i = tid; i < C; i += kFT) {
        const uint32_t key = s_ckey[i];
        const int jb = s_cj[i];
        if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
        else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
      }
    } else {
      for (int jb = tid; jb < nb; jb += kFT) {
        const uint32_t key = order_key(bs[jb]);
        if (b.bin(key) != bstar) continue;
        if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
        else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
      }
    }
    __syncthreads();
  }

  // ordered compaction (ties, in the radix path, admitted in ascending block order)
  const int wpt = (nw + kFT - 1) / kFT;
  const int w_lo = min(nw, tid * wpt), w_hi = min(nw, w_lo + wpt);
  uint32_t total;
  if (!ranked) {
    uint32_t ties = 0;
    for (int i = w_lo; i < w_hi; ++i) ties += __popc(s_tie[i]);
    uint32_t tie_before = block_exclusive_scan<kFT>(ties, s_scan, &total);
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
  uint32_t out_before = block_exclusive_scan<kFT>(sel_local, s_scan, &total);
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
  *reinterpret_cast<v4u*>(w.hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
}

}  // namespace

int64_t pool_ws_words(int chunks, int mm_cap) {
  const int64_t words = kHistBins + 2 * (int64_t)mm_cap + chunks + (int64_t)chunks * (kPoolChunk / 32) +
                        2 * (int64_t)chunks * kPoolChunkCand;
  return (words + 63) / 64 * 64;
}

hipError_t launch_pool_select(const PoolArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_q * a.chunks));
  if (!a.have_minmax) hipLaunchKernelGGL(k_pool_minmax, grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(k_pool_hist, grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(k_pool_mark, grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(k_pool_final, dim3((unsigned)a.n_q), dim3(kFT), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
