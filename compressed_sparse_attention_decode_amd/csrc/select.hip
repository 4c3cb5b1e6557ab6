// Top-P block pool selection (Full mode, second half).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (hierarchical sparse indexer: the
// Full layer keeps the Top-2048 blocks of 8 as the candidate pool).  Order is
// (block score descending, block id ascending); the pool is written in
// ascending block order.
//
// One 1024-thread workgroup per query, on order-preserving uint32 keys:
//  1. min/max pass: the bits above the highest bit where min and max differ
//     are common to every key, so the histograms start below them (keys of
//     similar scores share their top bits and would otherwise pile onto a few
//     LDS counters);
//  2. a 4096-bin LDS histogram of the next 12 bits gives the bin b* holding
//     the P-th best block;
//  3. one pass marks blocks in higher bins in an LDS bitmap (wave ballots)
//     and appends the blocks of bin b* to an LDS candidate list;
//  4. an exact radix select over the candidates' remaining bits finds the
//     threshold key T and how many blocks equal to T are still needed (a
//     candidate list that overflows LDS is re-read from global memory);
//  5. ordered compaction of the bitmap writes ascending block ids, admitting
//     blocks equal to T lowest id first.
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace csa2 {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kCandCap = 8192;
constexpr int kMaxWords = kMaxBlocks / 32;

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// keys agree on every bit >= lo (lo in [0, 32])
__device__ __forceinline__ bool same_above(uint32_t a, uint32_t b, int lo) {
  return ((uint64_t)a >> lo) == ((uint64_t)b >> lo);
}

// One pass over a query's block scores, 16-byte loads issued kU at a time
// (kU x 4 blocks per thread in flight).  f(jb0, key[4], valid-mask) sees
// blocks jb0 .. jb0+3; blocks >= nb are passed with their mask bit clear.
constexpr int kU = 8;
template <typename F>
__device__ __forceinline__ void sweep(const float* bs, int nb, F&& f) {
  const int tid = threadIdx.x;
  for (int base = 0; base < nb; base += kSelThreads * 4 * kU) {
    v4f x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jb0 = base + (u * kSelThreads + tid) * 4;
      x[u] = jb0 < nb ? *reinterpret_cast<const v4f*>(bs + jb0) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jb0 = base + (u * kSelThreads + tid) * 4;
      const int left = nb - jb0;
      const uint32_t vm = left >= 4 ? 15u : (left <= 0 ? 0u : (1u << left) - 1u);
      const uint32_t k[4] = {order_key(x[u][0]), order_key(x[u][1]), order_key(x[u][2]), order_key(x[u][3])};
      f(jb0, k, vm);
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void k_pool_select(PoolArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_sel[kMaxWords];
  __shared__ uint32_t s_tie[kMaxWords];
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int32_t s_cj[kCandCap];
  __shared__ uint32_t s_scan[kSelThreads / 64 + 1];
  __shared__ uint32_t s_misc[4];
  __shared__ uint32_t s_ccount;

  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);
  const int nb = (c + 7) >> 3;
  const int P = a.pool;
  int32_t* out = a.pool_blocks + (int64_t)q * P;
  if (nb <= P) {
    for (int j = tid; j < P; j += kSelThreads) out[j] = j < nb ? j : -1;
    if (tid == 0) a.pool_count[q] = nb;
    return;
  }
  const float* bs = a.bscore + (int64_t)q * a.ld;

  // 1. key range
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  sweep(bs, nb, [&](int, const uint32_t* k, uint32_t vm) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (vm >> e & 1u) { lo = min(lo, k[e]); hi = max(hi, k[e]); }
    }
  });
  const uint32_t kmin = block_min_u32<kSelThreads>(lo, s_scan);
  const uint32_t kmax = block_max_u32<kSelThreads>(hi, s_scan);
  const int top = highest_diff_bit(kmin, kmax);          // -1: all keys equal
  const int cs = max(0, top - 11);                        // coarse bins: bits [cs, top]
  const uint32_t cmask = top < 0 ? 0u : (uint32_t)((2ull << (top - cs)) - 1);

  // 2. coarse histogram and the bin b* of the P-th best block
  for (int i = tid; i < kHistBins; i += kSelThreads) s_hist[i] = 0;
  __syncthreads();
  sweep(bs, nb, [&](int, const uint32_t* k, uint32_t vm) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (vm >> e & 1u) atomicAdd(&s_hist[(k[e] >> cs) & cmask], 1u);
  });
  __syncthreads();
  constexpr int kPer = kHistBins / kSelThreads;
  uint32_t local = 0, cnt[kPer];
  for (int k = 0; k < kPer; ++k) {
    cnt[k] = s_hist[kHistBins - 1 - (tid * kPer + k)];
    local += cnt[k];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan<kSelThreads>(local, s_scan, &total);
  if (above < (uint32_t)P && (uint32_t)P <= above + local) {
    for (int k = 0; k < kPer; ++k) {
      if (above + cnt[k] >= (uint32_t)P) {
        s_misc[0] = kHistBins - 1 - (tid * kPer + k);
        s_misc[1] = above;
        break;
      }
      above += cnt[k];
    }
  }
  const int nw = (nb + 31) >> 5;
  for (int w = tid; w < nw; w += kSelThreads) s_tie[w] = 0;
  if (tid == 0) s_ccount = 0;
  __syncthreads();
  const uint32_t bstar = s_misc[0];
  uint32_t need = (uint32_t)P - s_misc[1];

  // 3. mark blocks above b* (a lane's 4 blocks form one nibble of the
  //    bitmap; 8 lanes OR their nibbles into a word), collect bin b*
  sweep(bs, nb, [&](int jb0, const uint32_t* k, uint32_t vm) {
    uint32_t hib = 0, cand = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t bin = (k[e] >> cs) & cmask;
      hib |= (uint32_t)((vm >> e & 1u) && bin > bstar) << e;
      cand |= (uint32_t)((vm >> e & 1u) && bin == bstar) << e;
    }
    uint32_t word = hib << (4 * (lane & 7));
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    word |= __shfl_xor(word, 4, 64);
    if ((lane & 7) == 0 && jb0 < nb) s_sel[jb0 >> 5] = word;
    // candidates: slot = wave base + per-element ballot prefixes
    uint64_t m[4];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[e] = __ballot(cand >> e & 1u);
      tot += (uint32_t)__popcll(m[e]);
    }
    if (tot == 0) return;
    uint32_t slot0 = 0;
    if (lane == 0) slot0 = atomicAdd(&s_ccount, tot);
    slot0 = __shfl(slot0, 0, 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (cand >> e & 1u) {
        const uint32_t slot = slot0 + lane_prefix(m[e]);
        if (slot < kCandCap) { s_ckey[slot] = k[e]; s_cj[slot] = jb0 + e; }
      }
      slot0 += (uint32_t)__popcll(m[e]);
    }
  });
  __syncthreads();
  const uint32_t C = s_ccount;
  const bool in_lds = C <= (uint32_t)kCandCap;

  // 4. radix select inside bin b* over bits [0, cs)
  uint32_t prefix = (uint32_t)(((uint64_t)kmin >> (top + 1)) << (top + 1)) | (bstar << cs);
  int fixed_lo = cs;                    // bits >= fixed_lo are decided
  while (fixed_lo > 0) {
    const int sh = max(0, fixed_lo - 8);
    const uint32_t dmask = (1u << (fixed_lo - sh)) - 1;
    for (int i = tid; i < 256; i += kSelThreads) s_hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (uint32_t i = tid; i < C; i += kSelThreads) {
        const uint32_t key = s_ckey[i];
        if (same_above(key, prefix, fixed_lo)) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
      }
    } else {
      for (int jb = tid; jb < nb; jb += kSelThreads) {
        const uint32_t key = order_key(bs[jb]);
        if (same_above(key, prefix, fixed_lo)) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
      }
    }
    __syncthreads();
    find_crossing(s_hist, 256, need, s_misc + 2);
    __syncthreads();
    prefix |= s_misc[2] << sh;
    need -= s_misc[3];
    fixed_lo = sh;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = need;

  // mark candidates above T (selected) and equal to T (tie bits)
  if (in_lds) {
    for (uint32_t i = tid; i < C; i += kSelThreads) {
      const uint32_t key = s_ckey[i];
      const int jb = s_cj[i];
      if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
      else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
    }
  } else {
    for (int jb = tid; jb < nb; jb += kSelThreads) {
      const uint32_t key = order_key(bs[jb]);
      if (((key >> cs) & cmask) != bstar) continue;
      if (key > T) atomicOr(&s_sel[jb >> 5], 1u << (jb & 31));
      else if (key == T) atomicOr(&s_tie[jb >> 5], 1u << (jb & 31));
    }
  }
  __syncthreads();

  // 5. ordered compaction; ties admitted in ascending block order
  const int wpt = (nw + kSelThreads - 1) / kSelThreads;
  const int w_lo = min(nw, tid * wpt), w_hi = min(nw, w_lo + wpt);
  uint32_t ties = 0;
  for (int w = w_lo; w < w_hi; ++w) ties += __popc(s_tie[w]);
  uint32_t tie_before = block_exclusive_scan<kSelThreads>(ties, s_scan, &total);
  uint32_t sel_local = 0;
  for (int w = w_lo; w < w_hi; ++w) {
    uint32_t t = s_tie[w], acc = 0;
    while (t && tie_before < need_eq) {
      const uint32_t bit = t & (0u - t);
      acc |= bit;
      t ^= bit;
      ++tie_before;
    }
    const uint32_t fin = s_sel[w] | acc;
    s_sel[w] = fin;
    sel_local += __popc(fin);
  }
  uint32_t out_before = block_exclusive_scan<kSelThreads>(sel_local, s_scan, &total);
  for (int w = w_lo; w < w_hi; ++w) {
    uint32_t fin = s_sel[w];
    while (fin) {
      const int b = __ffs(fin) - 1;
      fin &= fin - 1;
      if (out_before < (uint32_t)P) out[out_before] = w * 32 + b;
      ++out_before;
    }
  }
  if (tid == 0) a.pool_count[q] = P;
}

}  // namespace

hipError_t launch_pool_select(const PoolArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_pool_select, dim3(a.n_q), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
