// Block-wide helpers for the exact radix selections (1024-thread blocks).
#pragma once

#include "common.h"

namespace csa2 {

template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* sh) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = sh[0];
  for (int w = 1; w < NT / 64; ++w) r = min(r, sh[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = sh[0];
  for (int w = 1; w < NT / 64; ++w) r = max(r, sh[w]);
  __syncthreads();
  return r;
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
  uint32_t x = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
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

// Digit plan for a radix select over keys that all lie in [kmin, kmax]: the
// bits above the highest bit where kmin and kmax differ are common to every
// key, so the passes start there (this keeps the first histogram spread out).
struct DigitPlan {
  int top;        // highest differing bit, -1 if kmin == kmax
};

__device__ __forceinline__ int highest_diff_bit(uint32_t kmin, uint32_t kmax) {
  const uint32_t d = kmin ^ kmax;
  return d ? 31 - __clz(d) : -1;
}

}  // namespace csa2
