// The last step of a Full layer's Top-K taken from the Full scan's own
// position scores ("DeepSeek-V4.1-Flash 梗概" §3.2: a Full layer's index set
// comes from the query that scored the whole context): given the K best
// blocks of the pool, pick the K best of their positions by (score desc,
// position asc) and write them in ascending order, as Reindex writes its
// Top-K.  The blocks suffice: a block ranked above the block B of one of the
// K best positions p contributes its own maximum position, which ranks above
// p, so fewer than K blocks rank above B.
#pragma once

#include "common.h"
#include "radix_topk.h"
#include "select_common.h"

namespace csa2 {

// Called by all kTkThreads threads.  s_blk: the nsel selected block ids in
// ascending order (LDS); pk: the query's position keys (the scan's order
// keys, 0 for positions past the candidates), 8 per block; thread t takes
// blocks [BPT t, BPT (t + 1)) of the selection (nsel <= BPT * kTkThreads).
// Writes out[0 .. K) (ascending positions, -1 past the count), out_s (the
// scores) and *count, each optional, and the positions of ranks [r0, r1) to
// rows[rank - r0] (LDS, optional; ranks past the count are not written).
// Returns the count.
template <int BPT>
__device__ __forceinline__ uint32_t topk_positions(const int32_t* s_blk, uint32_t nsel, const uint32_t* pk, int K,
                                                   int32_t* out, float* out_s, int32_t* count, uint32_t* s_scan,
                                                   RadixLds& L, int32_t* rows = nullptr, int r0 = 0, int r1 = 0) {
  constexpr int PP = BPT * kBlock;                  // position slots per thread
  const int tid = threadIdx.x;
  uint32_t key[PP];
  int32_t mb[BPT];
  // (slots past the selection load block 0's keys, a valid row, and clear them)
#pragma unroll
  for (int b = 0; b < BPT; ++b) mb[b] = tid * BPT + b < (int)nsel ? s_blk[tid * BPT + b] : 0;
  v4u x0[BPT], x1[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    x0[b] = *reinterpret_cast<const v4u*>(pk + (int64_t)mb[b] * kBlock);
    x1[b] = *reinterpret_cast<const v4u*>(pk + (int64_t)mb[b] * kBlock + 4);
  }
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    const bool live = tid * BPT + b < (int)nsel;
    key[8 * b + 0] = live ? x0[b][0] : 0u; key[8 * b + 1] = live ? x0[b][1] : 0u;
    key[8 * b + 2] = live ? x0[b][2] : 0u; key[8 * b + 3] = live ? x0[b][3] : 0u;
    key[8 * b + 4] = live ? x1[b][0] : 0u; key[8 * b + 5] = live ? x1[b][1] : 0u;
    key[8 * b + 6] = live ? x1[b][2] : 0u; key[8 * b + 7] = live ? x1[b][3] : 0u;
  }
  const TopkCut cut = radix_topk<PP>(key, K, 0, L);
  uint32_t pflags = 0;
#pragma unroll
  for (int k = 0; k < PP; ++k) pflags |= (uint32_t)(key[k] >= cut.tt) << k;
  uint32_t total;
  uint32_t pos_before = block_exclusive_scan<kTkThreads>(__builtin_popcount(pflags), s_scan, &total);
#pragma unroll
  for (int k = 0; k < PP; ++k) {
    if (pflags >> k & 1u) {
      if (pos_before < (uint32_t)K) {
        const int32_t p = mb[k >> 3] * kBlock + (k & 7);
        if (out) out[pos_before] = p;
        if (out_s) out_s[pos_before] = key_float(key[k]);
        if (rows && (int)pos_before >= r0 && (int)pos_before < r1) rows[pos_before - r0] = p;
      }
      ++pos_before;
    }
  }
  if (out) {
    for (int t = (int)cut.keff + tid; t < K; t += kTkThreads) {
      out[t] = -1;
      if (out_s) out_s[t] = 0.0f;
    }
  }
  if (count && tid == 0) *count = (int32_t)cut.keff;
  return cut.keff;
}

}  // namespace csa2
