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
                                                   RadixLds& L, uint32_t floor, int32_t* rows = nullptr, int r0 = 0,
                                                   int r1 = 0) {
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
  // floor bounds the K-th best candidate block's key from below; that
  // block and the K - 1 above it each bring their best position, K distinct
  // keys at or above it, so the K-th best position key is too (with fewer
  // than K blocks no such bound holds)
  const TopkCut cut = radix_topk<PP, true>(key, K, 0, L, nsel >= (uint32_t)K ? floor : 0u);
  uint32_t pflags = 0;
#pragma unroll
  for (int k = 0; k < PP; ++k) pflags |= (uint32_t)(key[k] >= cut.tt) << k;
  uint32_t total;
  uint32_t pos_before = block_exclusive_scan<kTkThreads>(__builtin_popcount(pflags), s_scan, &total);
  if (out_s) {
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      if (pflags >> k & 1u) {
        if (pos_before + __builtin_popcount(pflags & ((1u << k) - 1u)) < (uint32_t)K)
          out_s[pos_before + __builtin_popcount(pflags & ((1u << k) - 1u))] = key_float(key[k]);
      }
    }
  }
  // the positions by rank into LDS (the histogram's words: free once the
  // selection is made), one short loop over this thread's selected slots;
  // then whole-row writes of the Top-K and of the rows [r0, r1)
  static_assert(kTkBins + kTkEmpty >= 2048, "a Top-K of up to 2048 positions staged in the histogram");
  uint32_t* s_tk = L.hist;
  uint32_t f = pflags;
  while (f) {
    const int k = __builtin_ctz(f);
    f &= f - 1;
    int32_t b = mb[0];
#pragma unroll
    for (int j = 1; j < BPT; ++j) b = (k >> 3) == j ? mb[j] : b;
    if (pos_before < (uint32_t)K) s_tk[pos_before] = (uint32_t)(b * kBlock + (k & 7));
    ++pos_before;
  }
  __syncthreads();
  const int keff = (int)cut.keff;
  if (out)
    for (int t = tid; t < K; t += kTkThreads) out[t] = t < keff ? (int32_t)s_tk[t] : -1;
  if (out_s)
    for (int t = keff + tid; t < K; t += kTkThreads) out_s[t] = 0.0f;
  if (rows)
    for (int t = r0 + tid; t < min(r1, keff); t += kTkThreads) rows[t - r0] = (int32_t)s_tk[t];
  if (count && tid == 0) *count = (int32_t)cut.keff;
  __syncthreads();                                   // (s_tk read before the caller reuses L)
  return cut.keff;
}

}  // namespace csa2
