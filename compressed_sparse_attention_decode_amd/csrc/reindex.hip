// Reindex: re-score only the candidate pool and keep the Top-K positions.
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (mode table: Reindex re-scores with
// this layer's indexer query and reuses the indexer keys of the last Full
// layer; hierarchical sparse indexer: later Reindex layers score only inside
// the 16,384-position pool and keep the Top-512) and §3 / §8 of the
// newsaint.id page (constant-size search domain; only the pool's keys are
// gathered).  Ties go to the lower position; output is ascending.
//
// One kernel, k_reindex, with 512-thread workgroups:
//  * scoring: one workgroup per 64 pool blocks of a query; a wave step
//    scores two pool blocks (16 positions, two contiguous key runs) with the
//    same contraction as the Full scan (fp8 rows: one fp8 MFMA per 16 heads
//    on the raw bytes; FP4 rows: f16 MFMAs), so the scores are the scan's
//    bit for bit.  Every key load of the
//    workgroup is issued before the first contraction (the work is short and
//    latency-bound).  Scores are written as order-preserving uint32 keys, 0
//    marking a slot that holds no candidate position;
//  * selection, by the last scoring workgroup of the query to finish: its
//    <= 16,384 keys sit in registers (32 consecutive pool slots per thread);
//    a radix select over (key - smallest key), whose first digit is the up
//    to 11 bits below the highest bit of the key range, finds the K-th
//    largest; the compaction runs in pool order (= ascending positions),
//    admitting keys equal to the threshold lowest position first.
//
// FP4 indexer rows (d = 128): a lane's 32 channels of a key are one 16-byte
// load of E2M1 codes and one dword holding its two E4M3 group scales; the
// query likewise.  Codes times scale are exact in f16.
#include "common.h"
#include "internal.h"
#include "radix_topk.h"
#include "select_common.h"
#include "topk_positions.h"
#include "pool_topk.h"

namespace csa2 {
namespace {

constexpr uint32_t kNoKeyRow = 0xFFFFFFFFu;   // a lane with no candidate position (paged rows)
constexpr uint32_t kNoKeyOff = 0xFFFFFF00u;   // a buffer offset past any plane: reads zero

// Scores of pool slots [i_begin, i_begin + BPW) of query q (8
// positions per slot) as order keys.  Slots past the pool count are scored
// too, from whatever block ids the row holds there (clamped to a zero key
// row): the selection masks them by the count, so nothing here waits for it.
template <int D, int HT, int NW, bool F4, int BPW>
__device__ __forceinline__ void score_part(const ReindexArgs& a, int q, int part) {
  static_assert(!F4 || D == 128, "FP4 rows are 128 channels wide");
  constexpr int KC = D / 32;
  constexpr int LB = F4 ? 16 : D / 4;              // key code bytes per lane per position
  constexpr int RB = F4 ? D / 2 : D;               // key code bytes per position
  constexpr int SB = D / 16;                       // FP4 scale bytes per position
  constexpr int SPW = BPW / (2 * NW);              // wave steps (2 blocks each) per wave
  static_assert(SPW * 2 * NW == BPW, "whole wave steps");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // known wave-uniform: no waterfall loops
  const int gq = lane >> 4, col = lane & 15;
  const int i_begin = part * BPW;
  const int i_end = min(a.pool, i_begin + BPW);
  // scalar loads issued together: one round trip
  const int n = load_uniform(a.n_visible + q);
  const int64_t sbase = load_uniform(a.seq_base + q);
  const int c = max(0, n - a.swa);
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;

  // pool entries of this wave's steps (step s covers pool slots
  // i_begin + 2s, +1; lane col>>3 picks the slot, col&7 the position)
  int pos[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) pos[u] = pool[min(i_begin + 2 * (wave + NW * u) + (col >> 3), a.pool - 1)];
  // the empty asm uses every loaded id, so the loads stay unconditional and
  // all in flight together (a load the compiler sinks into the masked
  // branch below waits on its own); the sequence base is waited for here
  // too, so its load is issued with the others
  asm volatile("" ::"s"(sbase));
#pragma unroll
  for (int u = 0; u < SPW; ++u) asm volatile("" : "+v"(pos[u]));
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = i_begin + 2 * (wave + NW * u) + (col >> 3);
    pos[u] = i < i_end ? pos[u] * kBlock + (col & 7) : c;
  }
  // every key load in flight at once (a position >= c reads zeros)
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    if (pos[u] > c || pos[u] < 0) pos[u] = c;
  }
  // the lane's key row: seq_base + p, or through the page table (one page id
  // per position, all loaded unconditionally from clamped slots before the
  // first use; a position with no candidate reads past the plane, zeros)
  uint32_t row[SPW];
  const bool paged = a.pages != nullptr;
  if (paged && c > 0) {
    int32_t pg[SPW];
    const uint32_t pmask = (1u << a.page_shift) - 1u;
#pragma unroll
    for (int u = 0; u < SPW; ++u) pg[u] = a.pages[sbase + (min(pos[u], c - 1) >> a.page_shift)];
#pragma unroll
    for (int u = 0; u < SPW; ++u) asm volatile("" : "+v"(pg[u]));
#pragma unroll
    for (int u = 0; u < SPW; ++u)
      row[u] = pos[u] < c ? ((uint32_t)pg[u] << a.page_shift) | ((uint32_t)pos[u] & pmask) : kNoKeyRow;
  } else {
#pragma unroll
    for (int u = 0; u < SPW; ++u) row[u] = paged ? kNoKeyRow : (uint32_t)pos[u];
  }
  const int64_t kbase = paged ? 0 : sbase;
  const uint32_t krows = paged ? (uint32_t)a.rows : (uint32_t)c;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.idx_k + kbase * RB, krows * RB);
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(F4 ? a.idx_k_scales + kbase * SB : a.idx_k, krows * SB);
  uint32_t kb[SPW][LB / 4];
  uint32_t ksw[SPW];                               // FP4: the dword holding the lane's two scales
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    // the Full scan's byte -> k-slot map (for d = 128 fp8 rows: chunks gq
    // and 4 + gq of 16 bytes), so both compute the same fp32 scores
    const uint32_t off = row[u] == kNoKeyRow ? kNoKeyOff : row[u] * RB + gq * (LB == 32 ? 16 : LB);
    const v4u x = buf_load16(rk, off);
    kb[u][0] = x[0]; kb[u][1] = x[1]; kb[u][2] = x[2]; kb[u][3] = x[3];
    if constexpr (F4) {
      ksw[u] = __builtin_amdgcn_raw_buffer_load_b32(
          rks, row[u] == kNoKeyRow ? kNoKeyOff : row[u] * SB + (gq >> 1) * 4, 0, 0);
    } else if constexpr (LB == 32) {
      const v4u y = buf_load16(rk, off + 64);
      kb[u][4] = y[0]; kb[u][5] = y[1]; kb[u][6] = y[2]; kb[u][7] = y[3];
    }
  }

  // query fragments: loads from clamped (valid) rows, padded heads zeroed
  v8h qf[HT][KC];
  float wv[HT][4];
  const uint8_t* qp = a.idx_q + (int64_t)q * a.hi * RB;
  uint32_t qraw[HT][KC][2];
  uint32_t qsw[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int hc = min(t * 16 + col, a.hi - 1);
    if constexpr (F4) {
      const v4u x = *reinterpret_cast<const v4u*>(qp + (int64_t)hc * RB + gq * 16);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qraw[t][kc][0] = x[kc];
      qsw[t] = *reinterpret_cast<const uint32_t*>(a.idx_q_scales + ((int64_t)q * a.hi + hc) * SB + (gq >> 1) * 4);
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int qb = D == 128 ? (kc >> 1) * 64 + gq * 16 + (kc & 1) * 8 : gq * 16 + kc * 8;
        const v2u x = *reinterpret_cast<const v2u*>(qp + (int64_t)hc * D + qb);
        qraw[t][kc][0] = x[0];
        qraw[t][kc][1] = x[1];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = a.idx_w[(int64_t)q * a.hi + min(t * 16 + gq * 4 + i, a.hi - 1)];
  }
  // every load above is issued before the first wait (the scheduler would
  // otherwise place later steps' key loads after the query conversion)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const bool live = t * 16 + col < a.hi;
    if constexpr (F4) {
      const v2h sc = fp4_pair_scales(qsw[t], gq & 1);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const _Float16 s = kc < 2 ? sc[0] : sc[1];
        qf[t][kc] = fp4x8_to_v8h(live ? qraw[t][kc][0] : 0u, v2h{s, s});
      }
    } else {
      // raw E4M3 bytes in the keys' byte -> k-slot map (qf[t][0], qf[t][1];
      // d = 64: the second half zero)
      const v4u lo = live ? v4u{qraw[t][0][0], qraw[t][0][1], qraw[t][1][0], qraw[t][1][1]} : v4u{0u, 0u, 0u, 0u};
      v4u hi = {0u, 0u, 0u, 0u};
      if constexpr (KC == 4)
        if (live) hi = v4u{qraw[t][2][0], qraw[t][2][1], qraw[t][3][0], qraw[t][3][1]};
      qf[t][0] = __builtin_bit_cast(v8h, lo);
      qf[t][1] = __builtin_bit_cast(v8h, hi);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = t * 16 + gq * 4 + i < a.hi ? wv[t][i] : 0.0f;
  }

  uint32_t* ks = a.keys + (int64_t)q * a.pool * kBlock;
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = i_begin + 2 * (wave + NW * u) + (col >> 3);
    // the key operand: f16 fragments (FP4 rows), or the raw E4M3 bytes
    // (d = 64: the second half zero)
    v8h kf[F4 ? KC : 1];
    v8i kr8 = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (F4) {
      const v2h sc = fp4_pair_scales(ksw[u], gq & 1);
      const v2h s0 = {sc[0], sc[0]}, s1 = {sc[1], sc[1]};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kf[kc] = fp4x8_to_v8h(kb[u][kc], kc < 2 ? s0 : s1);
    } else if constexpr (LB == 32) {
      kr8 = cat_v8i(v4u{kb[u][0], kb[u][1], kb[u][2], kb[u][3]}, v4u{kb[u][4], kb[u][5], kb[u][6], kb[u][7]});
    } else {
      kr8 = cat_v8i(v4u{kb[u][0], kb[u][1], kb[u][2], kb[u][3]}, v4u{0u, 0u, 0u, 0u});
    }
    // the Full scan's contraction and summation order: one fp8 MFMA per head
    // tile (fp8 rows) or four f16 ones (FP4 rows), four partial sums over the
    // head tiles, then the lane groups
    float pp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (F4) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[t][kc], kf[kc], acc, 0, 0, 0);
      } else {
        acc = mfma_fp8_k128(cat_v8i(__builtin_bit_cast(v4u, qf[t][0]), __builtin_bit_cast(v4u, qf[t][1])), kr8, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[i] += wv[t][i] * fmaxf(acc[i], 0.0f);
    }
    const float sum = sum_rows4((pp[0] + pp[1]) + (pp[2] + pp[3]));
    // order-preserving key; 0 marks a slot with no candidate position
    if (gq == 0 && i < i_end) ks[i * kBlock + (col & 7)] = pos[u] < c ? order_key(sum) : 0u;
  }
}

constexpr int kBlkPer = kPer / kBlock;             // pool blocks per selecting thread
static_assert(kMaxCand == 2048 * kBlock, "the largest pool's positions");

// The Top-K of the query's pool positions from the scoring workgroups' keys.
__device__ __forceinline__ void topk_select(const ReindexArgs& a, int q, int32_t b0, int32_t b1, int32_t b2,
                                            int32_t b3, int pcnt) {
  static_assert(kBlkPer == 4, "four pool blocks per thread");
  const int32_t blk[kBlkPer] = {b0, b1, b2, b3};
  __shared__ uint32_t s_scan[kTkWaves];
  const int tid = threadIdx.x;
  const int K = a.topk;
  const uint32_t* ks = a.keys + (int64_t)q * a.pool * kBlock;
  int32_t* out = a.topk_pos + (int64_t)q * K;
  float* out_s = a.topk_scores ? a.topk_scores + (int64_t)q * K : nullptr;

  // thread t holds slots [kPer t, kPer (t + 1)) (pool order = ascending
  // positions); blk holds the pool blocks they belong to.  The rows always
  // hold 8P keys: slots past the pool count are cleared.
  uint32_t key[kPer];
  const int s0 = tid * kPer;
  const bool mine = s0 < a.pool * kBlock;
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) {
    const v4u x = mine ? *reinterpret_cast<const v4u*>(ks + s0 + v * 4) : v4u{0u, 0u, 0u, 0u};
    key[4 * v] = x[0]; key[4 * v + 1] = x[1]; key[4 * v + 2] = x[2]; key[4 * v + 3] = x[3];
  }
  const int nh = pcnt * kBlock - s0;         // slots of this thread inside the pool count
  if (nh < kPer) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) key[k] = k < nh ? key[k] : 0u;
  }
  const TopkCut cut = radix_topk<kPer, true>(key, K);

  uint32_t flags = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) flags |= (uint32_t)(key[k] >= cut.tt) << k;
  uint32_t total;
  uint32_t before = block_exclusive_scan<kTkThreads>(__builtin_popcount(flags), s_scan, &total);
  if (!out_s) {
    // a thread holds about one selected key: visit only the set bits
    while (flags) {
      const int k = __builtin_ctz(flags);
      flags &= flags - 1;
      int32_t b = blk[0];
#pragma unroll
      for (int j = 1; j < kBlkPer; ++j) b = (k >> 3) == j ? blk[j] : b;
      if (before < (uint32_t)K) out[before] = b * kBlock + (k & 7);
      ++before;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (flags >> k & 1u) {
        if (before < (uint32_t)K) {
          out[before] = blk[k >> 3] * kBlock + (k & 7);
          out_s[before] = key_float(key[k]);
        }
        ++before;
      }
    }
  }
  for (int t = (int)cut.keff + tid; t < K; t += kTkThreads) {
    out[t] = -1;
    if (out_s) out_s[t] = 0.0f;
  }
  if (tid == 0) a.topk_count[q] = (int32_t)cut.keff;
}

// One kernel per Reindex call.  Every workgroup scores its BPW pool slots
// (64, or 128 when the grid would otherwise take several rounds); the last workgroup of a query to finish (a per-query counter in
// the workspace, left at zero for the next call) selects that query's Top-K
// from all of its keys.  The keys cross workgroups through memory: after a
// barrier, each workgroup's release fence publishes its stores before it
// counts itself in, and the last one's acquire fence makes the others'
// visible before it reads them.
template <int D, int HT, bool F4, int BPW>
__global__ __launch_bounds__(kTkThreads) void k_reindex(ReindexArgs a) {
  __shared__ uint32_t s_last;
  const int q = blockIdx.x / a.split, part = blockIdx.x % a.split;
  // the selection's pool blocks and count (inputs of this call) are loaded by
  // every workgroup before its scoring, so the last one has them at hand
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;
  const int j0 = (int)threadIdx.x * kBlkPer;
  const int32_t b0 = pool[min(j0, a.pool - 1)], b1 = pool[min(j0 + 1, a.pool - 1)];
  const int32_t b2 = pool[min(j0 + 2, a.pool - 1)], b3 = pool[min(j0 + 3, a.pool - 1)];
  const int pcnt = load_uniform(a.pool_count + q);
  score_part<D, HT, kTkWaves, F4, BPW>(a, q, part);
  if (a.score_only) return;             // the next kernel selects (its launch orders the keys)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's key stores have reached L2
  __syncthreads();
  if (threadIdx.x == 0) {
    // one release per workgroup (an L2 write-back), one acquire (an
    // invalidate) only in the last: per-wave fences would flush and drop the
    // L2 that the other workgroups are reading
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t prev = __hip_atomic_fetch_add(a.done + q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(a.split - 1);
    if (s_last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      a.done[q] = 0;
    }
  }
  __syncthreads();
  if (!s_last) return;
  topk_select(a, q, b0, b1, b2, b3, pcnt);
}

template <int D, bool F4, int BPW>
hipError_t launch_db(const ReindexArgs& a, hipStream_t s) {
  const int ht = (a.hi + 15) / 16;
  const dim3 grid((unsigned)(a.n_q * a.split)), block(kTkThreads);
  switch (ht) {
    case 1: hipLaunchKernelGGL((k_reindex<D, 1, F4, BPW>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_reindex<D, 2, F4, BPW>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_reindex<D, 3, F4, BPW>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_reindex<D, 4, F4, BPW>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int D, bool F4>
hipError_t launch_d(const ReindexArgs& a, hipStream_t s) {
  if (a.blocks_per_wg == kReindexBlocksHuge) return launch_db<D, F4, kReindexBlocksHuge>(a, s);
  if (a.blocks_per_wg == kReindexBlocksWide) return launch_db<D, F4, kReindexBlocksWide>(a, s);
  if (a.blocks_per_wg == kReindexBlocksNarrow) return launch_db<D, F4, kReindexBlocksNarrow>(a, s);
  return launch_db<D, F4, kReindexBlocks>(a, s);
}

// ---------------------------------------------------------------- Full layer
// A Full layer's Top-K from the Full scan's own scores ("DeepSeek-V4.1-Flash
// 梗概" §3.2: the Full layer takes its index set with the query that scored
// the whole context, so its Top-K inside the pool is Reindex with that same
// query).  The scan left every candidate position's score (as an order key)
// and every block's maximum; one workgroup per query then selects, with no
// key read and no re-scoring:
//  1. the K best blocks of the pool (by (block score desc, block id asc)).
//     Every one of the K best positions of the pool lies in them: a block
//     ranked above the block B of such a position p contributes its maximum
//     position, which ranks above p, so fewer than K blocks rank above B;
//  2. the K best positions of those blocks (by (score desc, position asc)),
//     written in ascending order, as Reindex writes them.
// Scores and ties are those of k_reindex (same contraction and summation
// order), so the result is the same set.
template <int BPT>
__global__ __launch_bounds__(kTkThreads) void k_topk_keys(TopkKeysArgs a) {
  __shared__ PoolTopkLds<BPT> s_sel;
  const int q = blockIdx.x;
  const int P = a.pool, K = a.topk;
  PoolTopkOut o;
  o.pool = nullptr;
  o.pool_count = nullptr;
  o.topk = a.topk_pos + (int64_t)q * K;
  o.topk_count = a.topk_count + q;
  o.rows = nullptr;
  o.r0 = o.r1 = 0;
  topk_from_pool<BPT>(a.pool_blocks + (int64_t)q * P, min(load_uniform(a.pool_count + q), P), P,
                      a.bscore + (int64_t)q * a.ld, a.pkey + (int64_t)q * a.ld_pkey, K, o,
                      a.topk_scores ? a.topk_scores + (int64_t)q * K : nullptr, s_sel, [] {});
}

}  // namespace

hipError_t launch_topk_keys(const TopkKeysArgs& a, hipStream_t s) {
  // blocks per thread for the K best blocks: K <= 512 -> 1, <= 1024 -> 2, else 4
  const dim3 grid((unsigned)a.n_q), block(kTkThreads);
  if (a.pool > 2048 || a.topk > 2048) return hipErrorInvalidValue;
  if (a.topk <= kTkThreads) hipLaunchKernelGGL(k_topk_keys<1>, grid, block, 0, s, a);
  else if (a.topk <= 2 * kTkThreads) hipLaunchKernelGGL(k_topk_keys<2>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_topk_keys<4>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reindex(const ReindexArgs& a, hipStream_t s) {
  if (a.idx_k_scales) {
    if (a.d != 128 || !a.idx_q_scales) return hipErrorInvalidValue;
    return launch_d<128, true>(a, s);
  }
  return a.d == 64 ? launch_d<64, false>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace csa2
