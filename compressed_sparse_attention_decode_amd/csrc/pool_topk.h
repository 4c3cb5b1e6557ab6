// The pool of a query with at most kMaxCand blocks, and optionally its Full
// layer's Top-K, selected by one 512-thread workgroup that holds all of the
// query's block keys in registers.
//
// Pool ("DeepSeek-V4.1-Flash 梗概" §3.1, the Full indexer keeps the P best
// blocks by block maximum): the radix Top-K of radix_topk.h over the block
// keys, ties to the lower block id, written in ascending order.
//
// Top-K (same page, §3.2: a Full layer's index set comes from the query that
// scored the whole context): the K best positions of the pool by (score
// desc, position asc), from the scan's position keys (topk_positions.h).
// Its candidate blocks are the pool's blocks at or above the lower edge of
// the first histogram's bin that holds the K-th best block: a superset of
// the K best blocks (ties to the lower id), so their positions hold the K
// best positions, and kept in ascending order so that slot order is
// position order for the ties.  Only when that bin is so crowded that the
// candidates exceed the BPT blocks per thread of the positions step does a
// second radix select pick exactly the K best blocks of the pool (the keys
// outside it cleared first).
#pragma once

#include "common.h"
#include "radix_topk.h"
#include "select_common.h"
#include "topk_positions.h"

namespace csa2 {

// Where the selection goes; every pointer is optional.
struct PoolTopkOut {
  int32_t* pool;         // [P] block ids ascending, -1 past the count
  int32_t* pool_count;
  int32_t* topk;         // [K] positions ascending, -1 past the count
  int32_t* topk_count;
  int32_t* rows;         // LDS: Top-K ranks [r0, r1) to rows[rank - r0]
  int r0, r1;
};

// The LDS of one selection (s_blk: BPT blocks per thread).
template <int BPT>
struct PoolTopkLds {
  RadixLds radix;
  int32_t blk[BPT > 0 ? kTkThreads * BPT : 1];
  uint32_t scan[kTkWaves];
};

// Called by all kTkThreads threads.  bs: the query's block scores (row
// stride ld, a multiple of 4 floats, >= 4), nb <= kMaxCand of them valid;
// pk: its position keys (BPT > 0).  after_keys() runs once the block keys
// are in registers, before the first selection (a caller's own loads then
// land while it runs without delaying the keys).  Without o.pool (the pool
// is written elsewhere) and with K <= P the Top-K needs no exact pool: the K
// best blocks lie in the pool, and the blocks at or above the first
// histogram's bound for the K-th block (radix_bound) are its candidates.
// Returns the Top-K count (BPT > 0) or the pool count.  Contains barriers.
template <int BPT, typename AfterKeys>
__device__ __forceinline__ uint32_t pool_topk_select(const float* bs, int ld, int nb, int P, int K,
                                                     const uint32_t* pk, const PoolTopkOut& o,
                                                     PoolTopkLds<BPT>& L, AfterKeys&& after_keys) {
  constexpr uint32_t kCap = kTkThreads * BPT;       // candidate blocks of the positions step
  const int tid = threadIdx.x;
  // thread t holds blocks [kPer t, kPer (t + 1)); the loads are bounded by
  // the row stride only, so they need not wait for the block count, which
  // masks them afterwards.  Every load is issued, clamped into the row, and
  // masked after it: a load under a condition would be waited for at once,
  // which made four round trips of the eight.
  const int s0 = tid * kPer;
  v4f x[kPer / 4];
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) x[v] = *reinterpret_cast<const v4f*>(bs + min(s0 + 4 * v, ld - 4));
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) {
    if (s0 + 4 * v >= ld) x[v] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  uint32_t key[kPer];
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * v + e] = s0 + 4 * v + e < nb ? order_key(x[v][e]) : 0u;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) asm volatile("" : "+v"(key[k]));   // the keys are complete here
  after_keys();
  if constexpr (BPT > 0) {
    if (!o.pool && !o.pool_count && K <= P) {
      const TopkBound bd = radix_bound<kPer>(key, K, L.radix);
      uint32_t cflags = 0;
#pragma unroll
      for (int k = 0; k < kPer; ++k) cflags |= (uint32_t)(key[k] >= bd.lb) << k;
      uint32_t ncand;
      uint32_t cb = block_exclusive_scan<kTkThreads>(__builtin_popcount(cflags), L.scan, &ncand);
      if (ncand <= kCap) {
        while (cflags) {
          const int k = __builtin_ctz(cflags);
          cflags &= cflags - 1;
          L.blk[cb++] = s0 + k;                    // ascending block ids
        }
        __syncthreads();
        return topk_positions<BPT>(L.blk, ncand, pk, K, o.topk, nullptr, o.topk_count, L.scan, L.radix, bd.lb,
                                   o.rows, o.r0, o.r1);
      }
      // (a crowded bin: the exact path below)
    }
  }
  const TopkCut cut = radix_topk<kPer>(key, P, BPT > 0 ? K : 0, L.radix);

  // pool members, and (BPT > 0) the candidate blocks of the Top-K: both
  // offsets from one block scan (16-bit fields: at most 16,384 of each)
  uint32_t flags = 0, cflags = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const bool in = key[k] >= cut.tt;
    flags |= (uint32_t)in << k;
    if constexpr (BPT > 0) cflags |= (uint32_t)(in && key[k] >= cut.lb2) << k;
  }
  uint32_t total;
  const uint32_t packed = block_exclusive_scan<kTkThreads>(
      __builtin_popcount(flags) | (uint32_t)__builtin_popcount(cflags) << 16, L.scan, &total);
  if (o.pool) {
    uint32_t before = packed & 0xFFFFu;
    while (flags) {
      const int k = __builtin_ctz(flags);
      flags &= flags - 1;
      if (before < (uint32_t)P) o.pool[before] = s0 + k;
      ++before;
    }
    for (int t = (int)cut.keff + tid; t < P; t += kTkThreads) o.pool[t] = -1;
  }
  if (o.pool_count && tid == 0) *o.pool_count = (int32_t)cut.keff;
  if constexpr (BPT == 0) {
    return cut.keff;
  } else {
    const uint32_t ncand = total >> 16;
    uint32_t nsel;
    if (ncand <= kCap) {
      uint32_t cb = packed >> 16;
      while (cflags) {
        const int k = __builtin_ctz(cflags);
        cflags &= cflags - 1;
        L.blk[cb++] = s0 + k;                      // ascending block ids
      }
      nsel = ncand;
    } else {
      // the exact K best blocks of the pool (all of it when K exceeds its
      // count)
#pragma unroll
      for (int k = 0; k < kPer; ++k) key[k] = key[k] >= cut.tt ? key[k] : 0u;
      const TopkCut bc = radix_topk<kPer>(key, K, 0, L.radix);
      uint32_t bflags = 0;
#pragma unroll
      for (int k = 0; k < kPer; ++k) bflags |= (uint32_t)(key[k] >= bc.tt) << k;
      uint32_t bb = block_exclusive_scan<kTkThreads>(__builtin_popcount(bflags), L.scan, &nsel);
      while (bflags) {
        const int k = __builtin_ctz(bflags);
        bflags &= bflags - 1;
        if (bb < kCap) L.blk[bb] = s0 + k;         // ascending block ids
        ++bb;
      }
      nsel = min(nsel, kCap);
    }
    __syncthreads();
    return topk_positions<BPT>(L.blk, nsel, pk, K, o.topk, nullptr, o.topk_count, L.scan, L.radix, cut.lb2, o.rows,
                               o.r0, o.r1);
  }
}

// A Full layer's Top-K of a pool selected before (csa2_index_pool's
// output): the K best blocks of the pool by (block score desc, block id asc),
// then the K best of their positions (topk_positions.h).  The blocks suffice
// for the same reason as above.  Called by all kTkThreads threads; pool: the
// query's P block ids ascending, pcnt valid; bs: its block scores; pk: its
// position keys.  o.pool / o.pool_count are not written; out_s (optional)
// receives the kept positions' scores.  Returns the Top-K count.
template <int BPT, typename AfterKeys>
__device__ __forceinline__ uint32_t topk_from_pool(const int32_t* pool, int pcnt, int P, const float* bs,
                                                   const uint32_t* pk, int K, const PoolTopkOut& o, float* out_s,
                                                   PoolTopkLds<BPT>& L, AfterKeys&& after_keys) {
  constexpr int PB = 2048 / kTkThreads;             // pool slots per thread (P <= 2048)
  const int tid = threadIdx.x;
  int32_t blk[PB];
#pragma unroll
  for (int k = 0; k < PB; ++k) blk[k] = pool[min(tid * PB + k, P - 1)];
#pragma unroll
  for (int k = 0; k < PB; ++k) asm volatile("" : "+v"(blk[k]));
  float bv[PB];
#pragma unroll
  for (int k = 0; k < PB; ++k) bv[k] = bs[tid * PB + k < pcnt ? max(blk[k], 0) : 0];
  uint32_t bkey[PB];
#pragma unroll
  for (int k = 0; k < PB; ++k) bkey[k] = tid * PB + k < pcnt ? order_key(bv[k]) : 0u;
#pragma unroll
  for (int k = 0; k < PB; ++k) asm volatile("" : "+v"(bkey[k]));   // the keys are complete here
  after_keys();
  const TopkCut bc = radix_topk<PB>(bkey, K, 0, L.radix);
  uint32_t flags = 0;
#pragma unroll
  for (int k = 0; k < PB; ++k) flags |= (uint32_t)(bkey[k] >= bc.tt) << k;
  uint32_t nsel;
  uint32_t before = block_exclusive_scan<kTkThreads>(__builtin_popcount(flags), L.scan, &nsel);
#pragma unroll
  for (int k = 0; k < PB; ++k)
    if (flags >> k & 1u) L.blk[before++] = blk[k];   // ascending: the pool is ascending
  __syncthreads();
  return topk_positions<BPT>(L.blk, nsel, pk, K, o.topk, out_s, o.topk_count, L.scan, L.radix, 0u, o.rows, o.r0,
                             o.r1);
}

// A Reindex layer's Top-K from the order keys its scoring kernel wrote (one
// per pool position, 0 = no candidate; "DeepSeek-V4.1-Flash 梗概" §3.2:
// Reindex re-scores the inherited pool with the layer's own indexer query
// and keeps the K best positions): the K best by (key desc, slot asc), slot
// order being ascending position order, written in ascending order.  The
// same selection as k_reindex's last workgroup.  Called by all kTkThreads
// threads; ks: the query's 8 P keys; pool: its P block ids, pcnt valid.
// o.pool / o.pool_count are not written.  Returns the Top-K count.
// s_stage: LDS for the 8 P keys (<= kMaxCand words): they are read with
// 16-byte loads that cover whole lines (thread t takes chunks 512 v + t) into
// 128-byte rows whose chunks are XOR-swizzled by the row, then each thread
// reads its own 32 consecutive keys back (slot order stays position order).
template <typename AfterKeys>
__device__ __forceinline__ uint32_t topk_from_keys(const uint32_t* ks, const int32_t* pool, int pcnt, int P, int K,
                                                   const PoolTopkOut& o, RadixLds& L, uint32_t* s_scan,
                                                   uint32_t* s_stage, AfterKeys&& after_keys) {
  constexpr int kBP = kPer / kBlock;                // pool blocks per thread
  static_assert(kPer == 32, "a thread's keys are one 128-byte row of the staging");
  const int tid = threadIdx.x;
  int32_t blk[kBP];
#pragma unroll
  for (int j = 0; j < kBP; ++j) blk[j] = pool[min(tid * kBP + j, P - 1)];
  const int s0 = tid * kPer;
  const bool mine = s0 < P * kBlock;
  {
    v4u x[kPer / 4];
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
      x[v] = *reinterpret_cast<const v4u*>(ks + min(4 * (kTkThreads * v + tid), P * kBlock - 4));
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) {
      const int i = kTkThreads * v + tid, r = i >> 3, c = i & 7;   // row r, chunk c
      *reinterpret_cast<v4u*>(s_stage + r * kPer + ((c ^ (r & 7)) << 2)) = x[v];
    }
  }
  __syncthreads();
  uint32_t key[kPer];
#pragma unroll
  for (int c = 0; c < kPer / 4; ++c) {
    const v4u x = *reinterpret_cast<const v4u*>(s_stage + tid * kPer + ((c ^ (tid & 7)) << 2));
    key[4 * c] = x[0]; key[4 * c + 1] = x[1]; key[4 * c + 2] = x[2]; key[4 * c + 3] = x[3];
  }
  const int nh = mine ? pcnt * kBlock - s0 : 0;    // slots of this thread inside the pool count
#pragma unroll
  for (int k = 0; k < kPer; ++k) key[k] = k < nh ? key[k] : 0u;
#pragma unroll
  for (int k = 0; k < kPer; ++k) asm volatile("" : "+v"(key[k]));   // the keys are complete here
  after_keys();
  const TopkCut cut = radix_topk<kPer, true>(key, K, 0, L);
  uint32_t flags = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) flags |= (uint32_t)(key[k] >= cut.tt) << k;
  uint32_t total;
  uint32_t before = block_exclusive_scan<kTkThreads>(__builtin_popcount(flags), s_scan, &total);
  // the positions by rank into LDS (the histogram's words, free once the
  // selection is made), then whole-row writes of the Top-K and of the rows
  uint32_t* s_tk = L.hist;
  while (flags) {
    const int k = __builtin_ctz(flags);
    flags &= flags - 1;
    int32_t b = blk[0];
#pragma unroll
    for (int j = 1; j < kBP; ++j) b = (k >> 3) == j ? blk[j] : b;
    if (before < (uint32_t)K) s_tk[before] = (uint32_t)(b * kBlock + (k & 7));
    ++before;
  }
  __syncthreads();
  const int keff = (int)cut.keff;
  if (o.topk)
    for (int t = tid; t < K; t += kTkThreads) o.topk[t] = t < keff ? (int32_t)s_tk[t] : -1;
  if (o.rows)
    for (int t = o.r0 + tid; t < min(o.r1, keff); t += kTkThreads) o.rows[t - o.r0] = (int32_t)s_tk[t];
  if (o.topk_count && tid == 0) *o.topk_count = (int32_t)cut.keff;
  __syncthreads();                                   // (s_tk read before the caller reuses L)
  return cut.keff;
}

}  // namespace csa2
