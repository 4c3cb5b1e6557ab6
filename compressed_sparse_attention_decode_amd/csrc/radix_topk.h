// Exact Top-K of up to 16,384 uint32 order keys held in the registers of one
// 512-thread workgroup (32 consecutive slots per thread; key 0 = empty slot),
// ties to the lower slot.  Used by the Reindex selection (keys = position
// scores) and by the pool selection of queries with at most 16,384 blocks
// (keys = block scores).
//
// The selection is a radix select over the keys offset by the smallest key:
// the first digit is the (up to) 11 bits below the highest bit of (max - min),
// so its bins are linear in the key and cover the occupied range.  The bin
// holding the keff-th largest key is narrowed by further digits until it holds
// at most kRankCap keys, which are then ranked exactly by (key desc, slot
// asc); a bin that is taken whole ends the search at once, and a run of equal
// keys that stays above kRankCap is cut at the right slot with a block scan.
// The result is a threshold (T, ST): keys above T, and keys equal to T at
// slots <= ST, are selected.  Every per-key pass is a few branch-free
// instructions: the workgroup runs on one CU, so its time is VALU issue over
// the 16,384 keys.
#pragma once

#include "common.h"
#include "select_common.h"

namespace csa2 {

constexpr int kTkThreads = 512;                    // 8 waves: up to 256 VGPRs per thread
constexpr int kMaxCand = 16384;                    // keys of one selection (8 x 2048)
constexpr int kPer = kMaxCand / kTkThreads;        // 32 keys per thread, in registers
constexpr int kTkBins = 2048;                      // radix digit: up to 11 bits
constexpr int kTkEmpty = 16;                       // bins past kTkBins that count empty slots
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kRankCap = 128;                      // candidates ranked exactly against each other (quadratic)
static_assert(kTkBins == 4 * kTkThreads, "one 16-byte histogram clear per thread");

// Wave 0 scans a kTkBins histogram from the top.  total = all counted keys,
// need = min(want, total).  Writes out[0] = the bin where the count from the
// top first reaches need, out[1] = keys in higher bins, out[2] = keys in that
// bin (out[0..2] only if need > 0), out[3] = need, out[4] = total.  Each lane
// owns 32 consecutive bins, read with 16-byte LDS loads.  Called by one whole
// wave.
__device__ __forceinline__ void crossing_2048(const uint32_t* hist, uint32_t want, uint32_t* out) {
  constexpr int kPB = kTkBins / 64;
  const int lane = threadIdx.x & 63;
  const int first = kTkBins - kPB * (lane + 1);     // lane 0 holds the highest bins
  uint32_t c[kPB];
#pragma unroll
  for (int v = 0; v < kPB / 4; ++v) {
    const v4u x = *reinterpret_cast<const v4u*>(hist + first + 4 * v);
    c[4 * v] = x[0]; c[4 * v + 1] = x[1]; c[4 * v + 2] = x[2]; c[4 * v + 3] = x[3];
  }
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < kPB; ++k) local += c[k];
  const uint32_t x = wave_incl_scan_u32(local);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  const uint32_t need = min(want, total);
  if (lane == 0) { out[3] = need; out[4] = total; }
  // the lane whose run holds the crossing; its bins go one per lane (highest
  // first) through a second wave scan
  const uint64_t hit = __ballot(need > 0 && x - local < need && need <= x);
  if (hit == 0) return;
  const int L = __builtin_ctzll(hit);
  const uint32_t above_l = (uint32_t)__builtin_amdgcn_readlane((int)(x - local), L);
  const int top = kTkBins - 1 - kPB * L;           // the run's highest bin
  const uint32_t v = lane < kPB ? hist[top - lane] : 0u;
  const uint32_t above = above_l + wave_incl_scan_u32(v) - v;
  if (lane < kPB && above < need && need <= above + v) {
    out[0] = top - lane;
    out[1] = above;
    out[2] = v;
  }
}

// One workgroup per query.  The selection is a radix select over the order
// keys offset by the query's smallest key: the first digit is the (up to) 11
// bits below the highest bit of (max - min), so its bins are linear in the key
// and cover the occupied range.  The bin holding the keff-th largest key is
// narrowed by further digits until it holds at most kRankCap keys, which are
// then ranked exactly by (key desc, slot asc); a bin that is taken whole ends
// the search at once, and a run of equal keys that stays above kRankCap is cut
// at the right slot by a block scan.  The result is a threshold (T, ST): keys
// above T, and keys equal to T at slots <= ST, are selected.  Every per-key
// pass is a few branch-free instructions: the workgroup runs on one CU, so
// its time is VALU issue over the 16,384 keys.
// What the caller needs to emit the selection: keff = min(K, valid keys),
// and each thread's selected keys are exactly those with key[k] >= tt (the
// thread straddling the tie cut has had its excluded equal keys cleared).
// With a second rank K2 > 0, lb2 is a lower bound of the K2-th largest key
// read off the first histogram (the lower edge of its bin; every key when
// K2 covers them all), and n2 counts the keys >= lb2, so n2 >= min(K2, valid
// keys).  Without one, lb2 = 0 and n2 = 0.
struct TopkCut {
  uint32_t keff;
  uint32_t tt;
  uint32_t lb2;
  uint32_t n2;
};

// The selection's LDS.  Calls may share one (a barrier always separates one
// call's last read from the next call's first write).
struct __align__(16) RadixLds {
  uint32_t hist[kTkBins + kTkEmpty];
  uint64_t cand[kRankCap];
  uint32_t red[2 * kTkWaves];
  uint32_t misc[8];
  uint32_t misc2[8];
};

// All 512 threads call this with their PER keys (PER <= 32; thread t holds
// slots [PER t, PER (t + 1)); slots past the valid range already 0).
// Contains barriers; K >= 1, K2 >= 0 (0: no second rank).  TOP (with K2 =
// 0): when K <= kTkThreads, only the keys at or above t0, the smallest of
// the threads' own largest keys, enter the histogram: t0 is at most the
// K-th largest key (the threads' largest keys are kTkThreads >= K distinct
// keys at or above it), and every later pass works inside the crossing bin,
// so the result is the same with far fewer LDS atomics.  (A thread without
// keys makes t0 = 0: every key enters.)  floor (TOP only, uniform): a lower
// bound of the K-th largest key that the caller knows; the keys below it
// stay out of the histogram as well.
template <int PER, bool TOP = false>
__device__ __forceinline__ TopkCut radix_topk(uint32_t (&key)[PER], int K, int K2, RadixLds& L,
                                              uint32_t floor = 0u) {
  static_assert(PER >= 1 && PER <= 32, "a 32-bit candidate mask per thread");
  uint32_t* s_hist = L.hist;
  uint64_t* s_cand = L.cand;
  uint32_t* s_red = L.red;
  uint32_t* s_misc = L.misc;
  uint32_t* s_misc2 = L.misc2;

  const int tid = threadIdx.x, lane = tid & 63;

  const int s0 = tid * PER;
  *reinterpret_cast<v4u*>(s_hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
  if (tid < kTkEmpty / 4) *reinterpret_cast<v4u*>(s_hist + kTkBins + 4 * tid) = v4u{0u, 0u, 0u, 0u};
  if (tid == 0) s_misc[5] = 0;

  // key range: key - 1 sends empty slots to the top for the minimum
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    lo = min(lo, key[k] - 1u);
    hi = max(hi, key[k]);
  }
  if constexpr (TOP) {
    // the waves' smallest thread maxima (read after the reduction's barriers)
    const uint32_t tm = wave_reduce_u32(hi, [](uint32_t x, uint32_t y) { return min(x, y); });
    if (lane == 0) s_misc2[tid >> 6] = tm;
    static_assert(kTkWaves <= 8, "one word per wave");
  }
  block_minmax_u32<kTkThreads>(&lo, &hi, s_red);   // its barriers also order the clears
  const uint32_t kmin = lo + 1u, kmax = hi;
  uint32_t base = kmin;                      // the histogram's lowest key
  if constexpr (TOP) {
    uint32_t t0 = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) t0 = min(t0, s_misc2[w]);
    if (K <= kTkThreads) base = max(kmin, t0);
    base = max(base, floor);
  }

  uint32_t keff = 0, lb2 = 0, n2 = 0;
  uint32_t T = 0xFFFFFFFFu;                  // threshold key (no finite score has it)
  int ST = 0x7FFFFFFF;                       // keys == T at slots <= ST are selected
  if (kmax != 0) {
    const uint32_t d = kmax - base;
    int shift = d ? max(0, 21 - (int)__clz(d)) : 0;    // (d >> shift) < 2^11
    if constexpr (TOP) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (key[k] >= base) atomicAdd(&s_hist[(key[k] - base) >> shift], 1u);
    } else {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const uint32_t b = (key[k] - base) >> shift;
        atomicAdd(&s_hist[key[k] != 0 ? b : kTkBins + (lane & (kTkEmpty - 1))], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) crossing_2048(s_hist, (uint32_t)K, s_misc);
    else if (tid < 128 && K2 > 0) crossing_2048(s_hist, (uint32_t)K2, s_misc2);
    __syncthreads();
    keff = s_misc[3];
    if (K2 > 0 && s_misc2[3] > 0) {
      lb2 = base + (s_misc2[0] << shift);
      n2 = s_misc2[1] + s_misc2[2];
    }
    uint32_t need = keff - s_misc[1];         // keys still to take from the crossing bin
    uint32_t cand = s_misc[2];
    uint32_t blo = base + (s_misc[0] << shift);    // the crossing bin is [blo, blo + 2^shift)

    // Rare: a crossing bin with more than kRankCap keys (clustered or equal
    // scores).  Further digits of (key - blo) narrow it.
    while (cand > (uint32_t)kRankCap && need < cand && shift > 0) {
      const int sh2 = max(0, shift - 11);
      __syncthreads();                        // the previous crossing is read
      *reinterpret_cast<v4u*>(s_hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
      __syncthreads();
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const uint32_t r = key[k] - blo;
        if ((r >> shift) == 0) atomicAdd(&s_hist[r >> sh2], 1u);
      }
      __syncthreads();
      if (tid < 64) crossing_2048(s_hist, need, s_misc);
      __syncthreads();
      blo += s_misc[0] << sh2;
      need -= s_misc[1];
      cand = s_misc[2];
      shift = sh2;
    }

    if (need == cand) {
      T = blo;                                // the crossing bin is taken whole
    } else if (cand <= (uint32_t)kRankCap) {
      // rank the candidates exactly: (key, ~slot) compared as one 64-bit value.
      // Gather: each thread marks its candidates, a wave scan and one LDS
      // atomic per wave give the offsets, then plain stores (no per-key
      // atomic round trip).
      const uint32_t bw = 1u << shift;
      uint32_t cm = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) cm |= (uint32_t)(key[k] - blo < bw) << k;
      const uint32_t nc = __builtin_popcount(cm);
      const uint32_t incl = wave_incl_scan_u32(nc);
      uint32_t wbase = 0;
      if (lane == 63 && incl) wbase = atomicAdd(&s_misc[5], incl);
      uint32_t idx = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63) + incl - nc;
      // only the slots where some lane of the wave has a candidate (a
      // wave-uniform index, so key[k] is a uniform-indexed register read)
      uint32_t any = wave_reduce_u32(cm, [](uint32_t x, uint32_t y) { return x | y; });
      any = (uint32_t)__builtin_amdgcn_readfirstlane((int)any);
      while (any) {
        const int k = __builtin_ctz(any);
        any &= any - 1;
        if (cm >> k & 1u) s_cand[idx++] = ((uint64_t)key[k] << 32) | (uint32_t)~(uint32_t)(s0 + k);
      }
      __syncthreads();
      // four threads per candidate, each comparing a quarter of the others
      const int ci_idx = tid >> 2, part = tid & 3;
      if (ci_idx < (int)cand) {
        const uint64_t ci = s_cand[ci_idx];
        uint32_t r = 0;
#pragma unroll 4
        for (uint32_t j = part; j < cand; j += 4) r += s_cand[j] > ci;
        r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        if (part == 0 && r == need - 1) { s_misc[6] = (uint32_t)(ci >> 32); s_misc[7] = ~(uint32_t)ci; }
      }
      __syncthreads();
      T = s_misc[6];
      ST = (int)s_misc[7];
    } else {
      // all bits fixed: more than kRankCap equal keys, taken lowest slot first
      T = blo;
      uint32_t eq = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) eq += key[k] == T;
      uint32_t total;
      uint32_t before = block_exclusive_scan<kTkThreads>(eq, s_red, &total);
      if (before < need && need <= before + eq) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          before += key[k] == T;
          if (key[k] == T && before == need) s_misc[7] = (uint32_t)(s0 + k);
        }
      }
      __syncthreads();
      ST = (int)s_misc[7];
    }
  }

  // Selected: key > T, or key == T at a slot <= ST.  A thread whose slots all
  // lie past ST compares against T + 1, the others against T; the one thread
  // that straddles ST first clears its keys equal to T past ST.
  const uint32_t Tt = s0 > ST ? T + 1u : T;
  if (s0 <= ST && ST < s0 + PER - 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k) key[k] = (key[k] == T && s0 + k > ST) ? 0u : key[k];
  }
  return TopkCut{keff, Tt, lb2, n2};
}

// The first pass of radix_topk alone: a lower bound lb of the K-th largest
// key (the lower edge of the first histogram's bin that holds it; every key
// when K covers them all) and n, the number of keys >= lb (n >= min(K,
// valid keys)).  No key is left out of {key >= lb} that the exact K largest
// hold.  With no valid key lb = 0xFFFFFFFF, n = 0.  Called by all kTkThreads
// threads; contains barriers.
struct TopkBound {
  uint32_t lb;
  uint32_t n;
};
template <int PER>
__device__ __forceinline__ TopkBound radix_bound(const uint32_t (&key)[PER], int K, RadixLds& L) {
  static_assert(PER >= 1 && PER <= 32, "PER keys per thread");
  uint32_t* s_hist = L.hist;
  const int tid = threadIdx.x, lane = tid & 63;
  *reinterpret_cast<v4u*>(s_hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
  if (tid < kTkEmpty / 4) *reinterpret_cast<v4u*>(s_hist + kTkBins + 4 * tid) = v4u{0u, 0u, 0u, 0u};
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    lo = min(lo, key[k] - 1u);
    hi = max(hi, key[k]);
  }
  block_minmax_u32<kTkThreads>(&lo, &hi, L.red);   // its barriers also order the clears
  const uint32_t kmin = lo + 1u, kmax = hi;
  if (kmax == 0) return TopkBound{0xFFFFFFFFu, 0u};
  const uint32_t d = kmax - kmin;
  const int shift = d ? max(0, 21 - (int)__clz(d)) : 0;   // (d >> shift) < 2^11, as radix_topk
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const uint32_t b = (key[k] - kmin) >> shift;
    atomicAdd(&s_hist[key[k] != 0 ? b : kTkBins + (lane & (kTkEmpty - 1))], 1u);
  }
  __syncthreads();
  if (tid < 64) crossing_2048(s_hist, (uint32_t)K, L.misc2);
  __syncthreads();
  const TopkBound r{kmin + (L.misc2[0] << shift), L.misc2[1] + L.misc2[2]};
  __syncthreads();                                   // (the next selection may reuse L at once)
  return r;
}

// radix_bound for K <= kTkThreads, with a prefilter: the smallest of the
// threads' own largest keys, t0, is at most the K-th largest key (the
// threads' largest keys are kTkThreads >= K distinct keys at or above it),
// so only the keys at or above t0 enter the histogram, whose bins then span
// [t0, max]: a few thousand LDS atomics instead of one per key, and finer
// bins where the bound falls.  (A thread without keys makes t0 = 0: every
// key enters, as in radix_bound.)  Same result contract as radix_bound.
template <int PER>
__device__ __forceinline__ TopkBound radix_bound_top(const uint32_t (&key)[PER], int K, RadixLds& L) {
  static_assert(PER >= 1 && PER <= 32, "PER keys per thread");
  constexpr int NW = kTkWaves;
  uint32_t* s_hist = L.hist;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  *reinterpret_cast<v4u*>(s_hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    lo = min(lo, key[k] - 1u);
    hi = max(hi, key[k]);
  }
  // block minimum of (key - 1), maximum of the keys, minimum of the threads'
  // maxima: one barrier pair (its barriers also order the clear)
  uint32_t t0 = hi;
  lo = wave_reduce_u32(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  t0 = wave_reduce_u32(t0, [](uint32_t x, uint32_t y) { return min(x, y); });
  hi = wave_reduce_u32(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) { L.red[wave] = lo; L.red[NW + wave] = hi; L.misc[wave & 7] = t0; }
  static_assert(NW <= 8, "one misc word per wave");
  __syncthreads();
  uint32_t rl = 0xFFFFFFFFu, rh = 0, rt = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NW; ++w) { rl = min(rl, L.red[w]); rh = max(rh, L.red[NW + w]); rt = min(rt, L.misc[w]); }
  __syncthreads();
  const uint32_t kmin = rl + 1u, kmax = rh;
  if (kmax == 0) return TopkBound{0xFFFFFFFFu, 0u};
  const uint32_t base = K <= kTkThreads ? max(kmin, rt) : kmin;
  const uint32_t d = kmax - base;
  const int shift = d ? max(0, 21 - (int)__clz(d)) : 0;   // (d >> shift) < 2^11
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (key[k] >= base) atomicAdd(&s_hist[(key[k] - base) >> shift], 1u);
  __syncthreads();
  if (tid < 64) crossing_2048(s_hist, (uint32_t)K, L.misc2);
  __syncthreads();
  const TopkBound r{base + (L.misc2[0] << shift), L.misc2[1] + L.misc2[2]};
  __syncthreads();                                   // (the next selection may reuse L at once)
  return r;
}

// The same with LDS of its own (one per PER).
template <int PER = kPer, bool TOP = false>
__device__ __forceinline__ TopkCut radix_topk(uint32_t (&key)[PER], int K, int K2 = 0) {
  __shared__ RadixLds s_radix;
  return radix_topk<PER, TOP>(key, K, K2, s_radix);
}

}  // namespace csa2
