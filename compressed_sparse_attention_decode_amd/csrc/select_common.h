// Block-wide helpers for the exact radix selections (1024-thread blocks).
#pragma once

#include "common.h"

namespace csa2 {

// Block-wide min and max of one uint32 per thread in one barrier pair
// (blockDim.x = NT, a multiple of 64; `sh` needs 2 NT/64 words).
template <int NT>
__device__ __forceinline__ void block_minmax_u32(uint32_t* lo, uint32_t* hi, uint32_t* sh) {
  constexpr int NW = NT / 64;
  const uint32_t l = wave_reduce_u32(*lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  const uint32_t h = wave_reduce_u32(*hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sh[wave] = l; sh[NW + wave] = h; }
  __syncthreads();
  uint32_t rl = 0xFFFFFFFFu, rh = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { rl = min(rl, sh[w]); rh = max(rh, sh[NW + w]); }
  __syncthreads();
  *lo = rl;
  *hi = rh;
}

// In a histogram of `nbins` (a multiple of 64, <= 4096) counts, wave 0 finds
// the bin where the running count from the top first reaches `need`.
// Writes {bin, count strictly above it} to out[0..1].  Other waves return.
__device__ __forceinline__ void find_crossing(const uint32_t* hist, int nbins, uint32_t need, uint32_t* out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = nbins / 64;
  uint32_t local = 0;
  for (int k = 0; k < per; ++k) local += hist[nbins - 1 - (lane * per + k)];
  const uint32_t x = wave_incl_scan_u32(local);
  uint32_t above = x - local;
  if (above < need && need <= x) {
    for (int k = 0; k < per; ++k) {
      const int b = nbins - 1 - (lane * per + k);
      const uint32_t cnt = hist[b];
      if (above + cnt >= need) {
        out[0] = (uint32_t)b;
        out[1] = above;
        break;
      }
      above += cnt;
    }
  }
}

// Radix passes over keys in [kmin, kmax] start below the highest bit where
// kmin and kmax differ: the bits above it are common to every key, so the
// first histogram stays spread out.
__device__ __forceinline__ int highest_diff_bit(uint32_t kmin, uint32_t kmax) {
  const uint32_t d = kmin ^ kmax;
  return d ? 31 - __clz(d) : -1;
}

}  // namespace csa2
