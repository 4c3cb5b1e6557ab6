// The pool and the Full layer's Top-K of a query with more blocks than one
// workgroup holds in registers (more than kMaxCand, i.e. contexts past
// 131,200 positions), selected by one 512-thread workgroup from the Full
// scan's group keys: the largest block key of every kGroupBlocks (16)
// consecutive blocks.
//
// The pool is the P best blocks by block maximum and a Full layer's Top-K the
// K best positions ("DeepSeek-V4.1-Flash 梗概" §3.1 and §3.2).  Both are
// reached exactly through supersets:
//  * the m-th best group key g_m is at most the m-th best block key (the m
//    best groups each hold a block at or above g_m, and those blocks are
//    distinct), and for the same reason at most the m-th best position key;
//  * so each of the P best blocks (each of the K best positions) has a key at
//    or above any lower bound lb of g_P (of g_K), and so has its group: the
//    groups at or above lb, and their blocks at or above lb, hold all of them.
// lb is the lower edge of the first radix histogram's bin that holds g_m
// (radix_bound); with fewer than m groups every block is a candidate.  When
// the candidates overflow their room (crowded or equal scores), an exact
// radix select that streams every block score decides instead: slower, and
// exact for any input.
#pragma once

#include "common.h"
#include "pool_topk.h"
#include "radix_topk.h"
#include "select_common.h"
#include "topk_positions.h"

namespace csa2 {

constexpr int kGroupPer = 16;                              // group keys per thread
constexpr int kMaxGroups = kTkThreads * kGroupPer;         // 8192 groups: 131,072 blocks
constexpr int kPoolGroupCap = 4096;                        // candidate groups of a pool selection
constexpr int kPoolCandCap = kTkThreads * kGroupPer;       // candidate blocks of a pool selection
constexpr int kPoolGpt = 2;                                // candidate groups per thread and round
static_assert(kGroupBlocks == 16, "a group's blocks are four 16-byte loads");

// Thread t's group keys, read coalesced: groups 4 (512 v + t) + e (v, e < 4;
// every load instruction covers whole lines once), 0 past ng.  Slot order is
// not group order: callers mark candidates in an LDS bitmap and compact it.
__device__ __forceinline__ int group_of(int v, int e) { return 4 * (kTkThreads * v + (int)threadIdx.x) + e; }

__device__ __forceinline__ void load_group_keys_c(const uint32_t* gk, int ng, int gcap, uint32_t (&key)[kGroupPer]) {
  v4u x[kGroupPer / 4];
#pragma unroll
  for (int v = 0; v < kGroupPer / 4; ++v) x[v] = *reinterpret_cast<const v4u*>(gk + min(group_of(v, 0), gcap - 4));
#pragma unroll
  for (int v = 0; v < kGroupPer / 4; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * v + e] = group_of(v, e) < ng ? x[v][e] : 0u;
  }
#pragma unroll
  for (int k = 0; k < kGroupPer; ++k) asm volatile("" : "+v"(key[k]));   // the keys are complete here
}

// Marks this thread's groups with key >= lb in s_bits (kMaxGroups / 32
// words, cleared before the caller's last barrier) and returns how many.
__device__ __forceinline__ uint32_t mark_groups(const uint32_t (&key)[kGroupPer], uint32_t lb, uint32_t* s_bits) {
  uint32_t n = 0;
#pragma unroll
  for (int v = 0; v < kGroupPer / 4; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (key[4 * v + e] >= lb && key[4 * v + e] != 0u) {
        const int g = group_of(v, e);
        atomicOr(&s_bits[g >> 5], 1u << (g & 31));
        ++n;
      }
    }
  }
  return n;
}

// The marked groups in ascending order into out[0 ..): threads t <
// kMaxGroups / 32 take bitmap word t.  Contains barriers (a block scan).
__device__ __forceinline__ void compact_groups(const uint32_t* s_bits, int32_t* out, uint32_t* s_scan) {
  const int tid = threadIdx.x;
  uint32_t w = tid < kMaxGroups / 32 ? s_bits[tid] : 0u;
  uint32_t total;
  uint32_t at = block_exclusive_scan<kTkThreads>((uint32_t)__builtin_popcount(w), s_scan, &total);
  while (w) {
    const int k = __builtin_ctz(w);
    w &= w - 1;
    out[at++] = tid * 32 + k;
  }
}

// The 16 block scores of group g (rows of stride ld, 16-byte aligned; blocks
// past the row are clamped into it and masked by the caller).
__device__ __forceinline__ void load_group_blocks(const float* bs, int64_t ld, int g, v4f (&x)[4]) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    x[v] = *reinterpret_cast<const v4f*>(bs + min((int64_t)g * kGroupBlocks + 4 * v, ld - 4));
}

// ------------------------------------------------------------ exact fallback
// The K best of the n block keys order_key(bs[i]) by (key desc, index asc),
// as a threshold: the keys above T, and the first need_eq keys equal to T in
// index order; keff = min(K, n) of them in all.  A radix select over three
// digits (bits 31-21, 20-10, 9-0), each a pass over every score.  bs: a row
// of stride >= n rounded up to 4.  Called by all kTkThreads threads; contains
// barriers.
struct StreamCut {
  uint32_t T;
  uint32_t need_eq;
  uint32_t keff;
};

__device__ __forceinline__ StreamCut stream_cut(const float* bs, int n, int K, RadixLds& L) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, need = (uint32_t)K, keff = 0;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int fixed = pass == 0 ? 32 : (pass == 1 ? 21 : 10);   // bits >= fixed are decided
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    __syncthreads();                                      // the previous crossing is read
    *reinterpret_cast<v4u*>(L.hist + 4 * tid) = v4u{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int i = 4 * tid; i < n; i += 4 * kTkThreads) {
      const v4f x = *reinterpret_cast<const v4f*>(bs + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = order_key(x[e]);
        if (i + e < n && ((uint64_t)k >> fixed) == ((uint64_t)prefix >> fixed)) atomicAdd(&L.hist[(k >> sh) & dmask], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) crossing_2048(L.hist, need, L.misc2);
    __syncthreads();
    if (pass == 0) {
      keff = L.misc2[3];
      need = keff;
      if (keff == 0) return StreamCut{0xFFFFFFFFu, 0u, 0u};
    }
    prefix |= L.misc2[0] << sh;
    need -= L.misc2[1];
  }
  __syncthreads();
  return StreamCut{prefix, need, keff};
}

// The selection of stream_cut in ascending index order: emit(rank, i) for
// each selected block i, rank being its place in that order (< keff).
// Chunks of 16 blocks per thread; one block scan per chunk.
template <typename Emit>
__device__ __forceinline__ void stream_emit(const float* bs, int n, const StreamCut& cut, uint32_t* s_scan,
                                            Emit&& emit) {
  const int tid = threadIdx.x;
  uint32_t gt_base = 0, eq_base = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += 16 * kTkThreads) {
    const int i0 = c0 + 16 * tid;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + 4 * v;
      if (i < n) {
        const v4f x = *reinterpret_cast<const v4f*>(bs + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = order_key(x[e]);
          gt |= (uint32_t)(i + e < n && k > cut.T) << (4 * v + e);
          eq |= (uint32_t)(i + e < n && k == cut.T) << (4 * v + e);
        }
      }
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kTkThreads>(
        (uint32_t)__builtin_popcount(gt) | (uint32_t)__builtin_popcount(eq) << 16, s_scan, &total);
    uint32_t g = gt_base + (before & 0xFFFFu), e = eq_base + (before >> 16);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (gt >> k & 1u) {
        emit(g + min(e, cut.need_eq), i0 + k);
        ++g;
      } else if (eq >> k & 1u) {
        if (e < cut.need_eq) emit(g + e, i0 + k);
        ++e;
      }
    }
    gt_base += total & 0xFFFFu;
    eq_base += total >> 16;
  }
}

// ------------------------------------------------------------ Top-K
// The Full layer's Top-K of a query with nb > kMaxCand blocks (nb <=
// kMaxGroups * kGroupBlocks), as pool_topk_select's Top-K: the candidate
// groups at or above the bound of the K-th group, their candidate blocks in
// ascending order, then the K best of their positions (topk_positions.h).
// BPT candidate groups per thread (at most 512 BPT of them) and 512 BPT
// candidate blocks; s_grp: LDS for 512 BPT group ids.  after_keys() runs once
// the group keys are in registers.  Returns the Top-K count.  Contains
// barriers.
template <int BPT, typename AfterKeys>
__device__ __forceinline__ uint32_t topk_from_groups(const uint32_t* gk, int gcap, const float* bs, int64_t ld,
                                                     int nb, const uint32_t* pk, int K, const PoolTopkOut& o,
                                                     PoolTopkLds<BPT>& L, int32_t* s_grp, uint32_t* s_bits,
                                                     AfterKeys&& after_keys) {
  static_assert(BPT >= 1 && BPT <= 4, "16 BPT block flags per thread in 64 bits");
  constexpr uint32_t kCap = kTkThreads * BPT;
  const int tid = threadIdx.x;
  const int ng = (nb + kGroupBlocks - 1) / kGroupBlocks;
  uint32_t key[kGroupPer];
  load_group_keys_c(gk, ng, gcap, key);
  after_keys();
  if (tid < kMaxGroups / 32) s_bits[tid] = 0u;           // (ordered by the bound's barriers)
  const TopkBound bd = K <= kTkThreads ? radix_bound_top<kGroupPer>(key, K, L.radix)
                                       : radix_bound<kGroupPer>(key, K, L.radix);
  const uint32_t lb = ng >= K ? bd.lb : 1u;               // too few groups: every block
  uint32_t ngc;
  block_exclusive_scan<kTkThreads>(mark_groups(key, lb, s_bits), L.scan, &ngc);   // (completes the marks)
  if (ngc <= kCap) {
    compact_groups(s_bits, s_grp, L.scan);                // ascending group ids
    __syncthreads();
    // thread t: candidate groups [BPT t, BPT (t + 1)), every load issued first
    int gid[BPT];
#pragma unroll
    for (int g = 0; g < BPT; ++g) gid[g] = tid * BPT + g < (int)ngc ? s_grp[tid * BPT + g] : -1;
    v4f x[BPT][4];
#pragma unroll
    for (int g = 0; g < BPT; ++g) load_group_blocks(bs, ld, max(gid[g], 0), x[g]);
    uint64_t bflags = 0;
#pragma unroll
    for (int g = 0; g < BPT; ++g) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = gid[g] * kGroupBlocks + 4 * v + e;
          const bool in = gid[g] >= 0 && b < nb && order_key(x[g][v][e]) >= lb;
          bflags |= (uint64_t)in << (16 * g + 4 * v + e);
        }
      }
    }
    uint32_t ncand;
    uint32_t cb = block_exclusive_scan<kTkThreads>((uint32_t)__builtin_popcountll(bflags), L.scan, &ncand);
    if (ncand <= kCap) {
#pragma unroll
      for (int g = 0; g < BPT; ++g) {
        uint32_t f = (uint32_t)(bflags >> (16 * g)) & 0xFFFFu;
        while (f) {
          const int k = __builtin_ctz(f);
          f &= f - 1;
          L.blk[cb++] = gid[g] * kGroupBlocks + k;        // ascending block ids
        }
      }
      __syncthreads();
      return topk_positions<BPT>(L.blk, ncand, pk, K, o.topk, nullptr, o.topk_count, L.scan, L.radix, lb, o.rows,
                                 o.r0, o.r1);
    }
  }
  // crowded: the exact K best blocks (K <= kCap), then their positions
  const StreamCut cut = stream_cut(bs, nb, K, L.radix);
  if (cut.keff) stream_emit(bs, nb, cut, L.scan, [&](uint32_t r, int i) { L.blk[r] = i; });
  __syncthreads();
  return topk_positions<BPT>(L.blk, cut.keff, pk, K, o.topk, nullptr, o.topk_count, L.scan, L.radix, lb, o.rows,
                             o.r0, o.r1);
}

// ------------------------------------------------------------ Top-K, short queries
// The Full layer's Top-K of a query of nb <= kMaxCand blocks for an
// attention workgroup (the pool is written elsewhere, K <= P): the blocks at
// or above the first histogram's bound for the K-th block key, in ascending
// order, then the K best of their positions.  The block scores are read
// coalesced (thread t takes blocks 4 (512 v + t) .. + 3, v < 8: each load
// instruction covers whole lines once; 32 consecutive blocks per thread made
// every instruction touch 64 lines and fetch each line eight times), so slot
// order is not block order: the candidates are marked in an LDS bitmap
// (s_bits, 512 words) and compacted in ascending order from it.  A crowded
// bin takes the exact streaming selection.  Returns the Top-K count.
// Thread t's keys of blocks 4 (512 v + t) + e (v < 8, e < 4) of a row of
// ld >= 4 block scores, 0 at or past nb: whole lines per load instruction.
__device__ __forceinline__ void load_block_keys_c(const float* bs, int64_t ld, int nb, uint32_t (&key)[kPer]) {
  constexpr int NV = kPer / 4;                       // 16-byte loads per thread
  const int tid = threadIdx.x;
  v4f x[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v)
    x[v] = *reinterpret_cast<const v4f*>(bs + min((int64_t)(4 * (kTkThreads * v + tid)), ld - 4));
#pragma unroll
  for (int v = 0; v < NV; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * v + e] = 4 * (kTkThreads * v + tid) + e < nb ? order_key(x[v][e]) : 0u;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) asm volatile("" : "+v"(key[k]));   // the keys are complete here
}

template <int BPT, typename AfterKeys>
__device__ __forceinline__ uint32_t topk_from_blocks(const float* bs, int ld, int nb, const uint32_t* pk, int K,
                                                     const PoolTopkOut& o, PoolTopkLds<BPT>& L, uint32_t* s_bits,
                                                     AfterKeys&& after_keys) {
  constexpr uint32_t kCap = kTkThreads * BPT;
  constexpr int NV = kPer / 4;                       // 16-byte loads per thread
  const int tid = threadIdx.x;
  uint32_t key[kPer];
  load_block_keys_c(bs, ld, nb, key);
  after_keys();
  s_bits[tid] = 0u;                                  // (ordered by the bound's barriers)
  const TopkBound bd = K <= kTkThreads ? radix_bound_top<kPer>(key, K, L.radix) : radix_bound<kPer>(key, K, L.radix);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (key[4 * v + e] >= bd.lb) {
        const int b = 4 * (kTkThreads * v + tid) + e;
        atomicOr(&s_bits[b >> 5], 1u << (b & 31));
      }
    }
  }
  __syncthreads();
  // thread t: the bitmap word of blocks [32 t, 32 t + 32), compacted in
  // ascending order (only while within the room; the total decides)
  uint32_t w = s_bits[tid];
  uint32_t nsel;
  uint32_t cb = block_exclusive_scan<kTkThreads>((uint32_t)__builtin_popcount(w), L.scan, &nsel);
  if (nsel <= kCap) {
    while (w) {
      const int k = __builtin_ctz(w);
      w &= w - 1;
      L.blk[cb++] = tid * 32 + k;                    // ascending block ids
    }
  } else {
    // crowded: the exact K best blocks (K <= kCap), ascending
    const StreamCut cut = stream_cut(bs, nb, K, L.radix);
    if (cut.keff) stream_emit(bs, nb, cut, L.scan, [&](uint32_t r, int i) { L.blk[r] = i; });
    nsel = cut.keff;
  }
  __syncthreads();
  return topk_positions<BPT>(L.blk, nsel, pk, K, o.topk, nullptr, o.topk_count, L.scan, L.radix, bd.lb, o.rows,
                             o.r0, o.r1);
}

// ------------------------------------------------------------ pool
// The LDS of pool_from_groups.
struct PoolGroupLds {
  RadixLds radix;
  uint32_t scan[kTkWaves];
  uint32_t bits[kMaxGroups / 32];
  int32_t grp[kPoolGroupCap];
  uint32_t ckey[kPoolCandCap];
  int32_t cblk[kPoolCandCap];
};

// The pool of a query with nb > kMaxCand blocks (nb <= kMaxGroups *
// kGroupBlocks, P <= kPoolGroupCap / 2): the P best blocks by (key desc,
// block asc), written ascending to pool[0 .. P) (-1 past the count) with the
// count.  The candidate groups at or above the bound of the P-th group are
// read kPoolGpt per thread at a time; their blocks at or above the bound are
// listed in ascending order and ranked by radix_topk.  With fewer groups
// than P (nb < 16 P) the bound comes from the first kMaxCand blocks' keys
// instead: the P-th best key of any kMaxCand >= P of the blocks is at most
// the P-th best of all, and at nb <= 2 kMaxCand about 2P blocks reach it
// (every block was a candidate before, and the exact streaming selection
// over all of them ran).  Returns the count.  Contains barriers.
__device__ __forceinline__ uint32_t pool_from_groups(const uint32_t* gk, int gcap, const float* bs, int64_t ld, int nb,
                                                     int P, int32_t* pool, int32_t* pool_count, PoolGroupLds& L) {
  const int tid = threadIdx.x;
  const int ng = (nb + kGroupBlocks - 1) / kGroupBlocks;
  uint32_t key[kGroupPer];
  load_group_keys_c(gk, ng, gcap, key);
  if (tid < kMaxGroups / 32) L.bits[tid] = 0u;          // (ordered by the bound's barriers)
  uint32_t lb;
  if (ng >= P) {
    lb = radix_bound<kGroupPer>(key, P, L.radix).lb;
  } else {
    uint32_t bk[kPer];
    load_block_keys_c(bs, ld, kMaxCand, bk);             // nb > kMaxCand: every slot valid
    lb = radix_bound<kPer>(bk, P, L.radix).lb;
  }
  uint32_t ngc;
  block_exclusive_scan<kTkThreads>(mark_groups(key, lb, L.bits), L.scan, &ngc);   // (completes the marks)
  uint32_t ncand = 0;
  bool fast = ngc <= (uint32_t)kPoolGroupCap;
  if (fast) {
    compact_groups(L.bits, L.grp, L.scan);               // ascending group ids
    __syncthreads();
#pragma unroll 1
    for (int r0 = 0; r0 < (int)ngc; r0 += kPoolGpt * kTkThreads) {
      int gid[kPoolGpt];
#pragma unroll
      for (int g = 0; g < kPoolGpt; ++g) {
        const int idx = r0 + kPoolGpt * tid + g;
        gid[g] = idx < (int)ngc ? L.grp[idx] : -1;
      }
      v4f x[kPoolGpt][4];
#pragma unroll
      for (int g = 0; g < kPoolGpt; ++g) load_group_blocks(bs, ld, max(gid[g], 0), x[g]);
      uint32_t kk[kPoolGpt * kGroupBlocks];
      uint32_t f = 0;
#pragma unroll
      for (int g = 0; g < kPoolGpt; ++g) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 16 * g + 4 * v + e;
            kk[k] = order_key(x[g][v][e]);
            f |= (uint32_t)(gid[g] >= 0 && gid[g] * kGroupBlocks + 4 * v + e < nb && kk[k] >= lb) << k;
          }
        }
      }
      uint32_t tot;
      uint32_t w = ncand + block_exclusive_scan<kTkThreads>((uint32_t)__builtin_popcount(f), L.scan, &tot);
#pragma unroll
      for (int k = 0; k < kPoolGpt * kGroupBlocks; ++k) {
        if (f >> k & 1u) {
          if (w < (uint32_t)kPoolCandCap) {
            L.ckey[w] = kk[k];
            L.cblk[w] = gid[k >> 4] * kGroupBlocks + (k & 15);   // ascending block ids
          }
          ++w;
        }
      }
      ncand += tot;
    }
    __syncthreads();
    fast = ncand <= (uint32_t)kPoolCandCap;
  }
  uint32_t keff;
  if (fast) {
    uint32_t ck[kGroupPer];                               // candidate slots [16 t, 16 t + 16)
#pragma unroll
    for (int k = 0; k < kGroupPer; ++k) {
      const uint32_t s = (uint32_t)(tid * kGroupPer + k);
      ck[k] = s < ncand ? L.ckey[s] : 0u;
    }
    const TopkCut cut = radix_topk<kGroupPer>(ck, P, 0, L.radix);
    uint32_t fl = 0;
#pragma unroll
    for (int k = 0; k < kGroupPer; ++k) fl |= (uint32_t)(ck[k] >= cut.tt) << k;
    uint32_t tot;
    uint32_t before = block_exclusive_scan<kTkThreads>((uint32_t)__builtin_popcount(fl), L.scan, &tot);
#pragma unroll
    for (int k = 0; k < kGroupPer; ++k) {
      if (fl >> k & 1u) {
        if (before < (uint32_t)P) pool[before] = L.cblk[tid * kGroupPer + k];
        ++before;
      }
    }
    keff = cut.keff;
  } else {
    // crowded: exact by streaming every block score
    const StreamCut cut = stream_cut(bs, nb, P, L.radix);
    if (cut.keff) stream_emit(bs, nb, cut, L.scan, [&](uint32_t r, int i) { pool[r] = i; });
    keff = cut.keff;
  }
  for (int t = (int)keff + tid; t < P; t += kTkThreads) pool[t] = -1;
  if (tid == 0) *pool_count = (int32_t)keff;
  return keff;
}

}  // namespace csa2
