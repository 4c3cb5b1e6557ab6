// Reindex: re-score only the candidate pool and keep the Top-K positions.
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (mode table: Reindex re-scores with
// this layer's indexer query and reuses the indexer keys of the last Full
// layer; hierarchical sparse indexer: later Reindex layers score only inside
// the 16,384-position pool and keep the Top-512) and §3 / §8 of the
// newsaint.id page (constant-size search domain; only the pool's keys are
// gathered).  Ties go to the lower position; output is ascending.
//
// Two kernels:
//  * k_reindex_score: one workgroup per 32 pool blocks of a query; a wave
//    step scores two pool blocks (16 positions, two contiguous key runs) with
//    the same f16-MFMA contraction as the Full scan.  Every key load of the
//    workgroup is issued before the first contraction (the kernel is short
//    and latency-bound).  Scores are written as order-preserving uint32 keys,
//    0 marking a slot that holds no candidate position;
//  * k_topk_select: one 512-thread workgroup per query keeps its <= 16,384
//    keys in registers (32 consecutive pool slots per thread), finds the K-th
//    largest with a radix select of up to 11-bit digits starting at the
//    highest bit where the smallest and largest key differ (common leading
//    bits would pile every key onto one counter), and compacts in pool order
//    (= ascending positions), admitting keys equal to the threshold lowest
//    position first.
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace csa2 {
namespace {

template <int D, int HT>
__global__ __launch_bounds__(256) void k_reindex_score(ReindexArgs a) {
  constexpr int KC = D / 32;
  constexpr int LB = D / 4;                 // key bytes per lane per position
  constexpr int SPW = kReindexBlocks / 8;   // wave steps (2 blocks each) per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;
  const int q = blockIdx.x / a.split, part = blockIdx.x % a.split;
  const int cnt = a.pool_count[q];
  const int i_begin = part * kReindexBlocks;
  const int i_end = min(cnt, i_begin + kReindexBlocks);
  if (i_begin >= i_end) return;
  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;

  // pool entries of this wave's steps (step s covers pool slots
  // i_begin + 2s, +1; lane col>>3 picks the slot, col&7 the position)
  int pos[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = i_begin + 2 * (wave + 4 * u) + (col >> 3);
    pos[u] = i < i_end ? pool[i] * kBlock + (col & 7) : c;
  }
  // every key load in flight at once (a position >= c reads zeros)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.idx_k + a.seq_base[q] * D, (uint32_t)c * D);
  uint32_t kb[SPW][LB / 4];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    if (pos[u] > c || pos[u] < 0) pos[u] = c;
    const uint32_t off = (uint32_t)pos[u] * D + gq * LB;
    const v4u x = buf_load16(rk, off);
    kb[u][0] = x[0]; kb[u][1] = x[1]; kb[u][2] = x[2]; kb[u][3] = x[3];
    if constexpr (LB == 32) {
      const v4u y = buf_load16(rk, off + 16);
      kb[u][4] = y[0]; kb[u][5] = y[1]; kb[u][6] = y[2]; kb[u][7] = y[3];
    }
  }

  // query fragments: loads from clamped (valid) rows, padded heads zeroed
  v8h qf[HT][KC];
  float wv[HT][4];
  const uint8_t* qp = a.idx_q + (int64_t)q * a.hi * D;
  uint32_t qraw[HT][KC][2];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int hc = min(t * 16 + col, a.hi - 1);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const v2u x = *reinterpret_cast<const v2u*>(qp + (int64_t)hc * D + gq * LB + kc * 8);
      qraw[t][kc][0] = x[0];
      qraw[t][kc][1] = x[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = a.idx_w[(int64_t)q * a.hi + min(t * 16 + gq * 4 + i, a.hi - 1)];
  }
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const bool live = t * 16 + col < a.hi;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[t][kc] = fp8x8_to_v8h(live ? qraw[t][kc][0] : 0u, live ? qraw[t][kc][1] : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = t * 16 + gq * 4 + i < a.hi ? wv[t][i] : 0.0f;
  }

  uint32_t* ks = a.keys + (int64_t)q * a.pool * kBlock;
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = i_begin + 2 * (wave + 4 * u) + (col >> 3);
    if (i_begin + 2 * (wave + 4 * u) >= i_end) break;              // wave-uniform
    v8h kf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kf[kc] = fp8x8_to_v8h(kb[u][2 * kc], kb[u][2 * kc + 1]);
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[t][kc], kf[kc], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += wv[t][i] * fmaxf(acc[i], 0.0f);
    }
    sum = sum_rows4(sum);
    // order-preserving key; 0 marks a slot with no candidate position
    if (gq == 0 && i < i_end) ks[i * kBlock + (col & 7)] = pos[u] < c ? order_key(sum) : 0u;
  }
}

constexpr int kTkThreads = 512;                    // 8 waves: up to 256 VGPRs per thread
constexpr int kMaxCand = 2048 * kBlock;
constexpr int kPer = kMaxCand / kTkThreads;        // 32 keys per thread, in registers
constexpr int kBlkPer = kPer / kBlock;             // pool blocks per thread
constexpr int kTkBins = 2048;                      // radix digit: up to 11 bits
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kRankCap = 128;                     // candidates ranked exactly against each other (quadratic)

// Wave 0 finds, in a kTkBins histogram, the bin where the count from the top
// first reaches `need`: out[0] = bin, out[1] = keys in higher bins,
// out[2] = keys in the bin.  Each lane owns 32 bins; both passes over them
// are branch-free runs of independent LDS reads.
__device__ __forceinline__ void crossing_2048(const uint32_t* hist, uint32_t need, uint32_t* out) {
  constexpr int kPB = kTkBins / 64;
  const int lane = threadIdx.x;
  const uint32_t* h = hist + kTkBins - kPB * (lane + 1);      // the lane's bins, ascending
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < kPB; ++k) local += h[k];
  const uint32_t x = wave_incl_scan_u32(local);
  if (x - local < need && need <= x) {
    uint32_t above = x - local;            // keys in bins above the lane's run
#pragma unroll
    for (int k = kPB - 1; k >= 0; --k) {   // from the lane's highest bin down
      const uint32_t c = h[k];
      if (above < need && need <= above + c) {
        out[0] = kTkBins - kPB * (lane + 1) + k;
        out[1] = above;
        out[2] = c;
      }
      above += c;
    }
  }
}

__global__ __launch_bounds__(kTkThreads) void k_topk_select(ReindexArgs a) {
  __shared__ uint32_t s_hist[kTkBins + 1];          // + a bin that collects empty slots
  __shared__ uint64_t s_cand[kRankCap];
  __shared__ uint32_t s_red[3 * kTkWaves];
  __shared__ uint32_t s_scan[kTkWaves];
  __shared__ uint32_t s_misc[4];

  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.topk;
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;
  const uint32_t* ks = a.keys + (int64_t)q * a.pool * kBlock;
  int32_t* out = a.topk_pos + (int64_t)q * K;
  float* out_s = a.topk_scores ? a.topk_scores + (int64_t)q * K : nullptr;

  // thread t holds slots [kPer t, kPer (t + 1)) (pool order = ascending
  // positions) and the pool blocks they belong to.  The loads do not wait for
  // the pool count (the rows always hold 8P keys and P blocks): slots past
  // the count are masked once it arrives.  Empty slots are key 0.
  uint32_t key[kPer];
  int32_t blk[kBlkPer];
  const bool mine = tid * kPer < a.pool * kBlock;
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) {
    const int i = tid * kPer + v * 4;
    const v4u x = mine ? *reinterpret_cast<const v4u*>(ks + i) : v4u{0u, 0u, 0u, 0u};
    key[4 * v] = x[0]; key[4 * v + 1] = x[1]; key[4 * v + 2] = x[2]; key[4 * v + 3] = x[3];
  }
#pragma unroll
  for (int j = 0; j < kBlkPer; ++j) blk[j] = mine ? pool[tid * kBlkPer + j] : 0;
  const int N = a.pool_count[q] * kBlock;
  for (int i = tid; i <= kTkBins; i += kTkThreads) s_hist[i] = 0;
  if (tid == 0) s_misc[3] = 0;

  // count of valid keys, their min and max (branch-free; one barrier)
  uint32_t nvalid = 0, lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    key[k] = tid * kPer + k < N ? key[k] : 0u;
    nvalid += key[k] != 0;
    lo = min(lo, key[k] != 0 ? key[k] : 0xFFFFFFFFu);
    hi = max(hi, key[k]);
  }
  nvalid = wave_reduce_u32(nvalid, [](uint32_t x, uint32_t y) { return x + y; });
  lo = wave_reduce_u32(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  hi = wave_reduce_u32(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) {
    s_red[wave] = nvalid;
    s_red[kTkWaves + wave] = lo;
    s_red[2 * kTkWaves + wave] = hi;
  }
  __syncthreads();
  uint32_t total = 0, kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    total += s_red[w];
    kmin = min(kmin, s_red[kTkWaves + w]);
    kmax = max(kmax, s_red[2 * kTkWaves + w]);
  }
  const uint32_t keff = min((uint32_t)K, total);

  // Selection.  A histogram over kTkBins linear bins of the score range
  // [min, max] (monotone in the key, and spread evenly, unlike bit digits of
  // scores that share an exponent) gives the bin b1 holding the keff-th
  // largest key.  Its keys are the candidates: up to kRankCap of them are
  // ranked exactly against each other by (key desc, slot asc), which also
  // settles ties, and the selected set is {key > T} plus {key == T, slot <=
  // ST}.  More candidates: radix digits of up to 11 bits over the candidates'
  // own key range narrow them first; a long run of equal keys falls back to
  // admitting equal keys lowest slot first with a block scan.
  int64_t T = 0;
  int ST = -1;                // with T: keys == T at slots <= ST are taken
  uint32_t need_eq = 0;       // fallback: need_eq keys == T, lowest slots first
  bool by_scan = false;
  if (keff > 0) {
    const float flo = key_float(kmin), fhi = key_float(kmax);
    float scale = (float)kTkBins / (fhi - flo);
    if (!(scale > 0.0f && scale < 3.0e38f)) scale = 0.0f;    // all keys equal (or a huge range)
    auto lbin = [&](uint32_t k) { return min((int)((key_float(k) - flo) * scale), kTkBins - 1); };
#pragma unroll
    for (int k = 0; k < kPer; ++k) atomicAdd(&s_hist[key[k] != 0 ? lbin(key[k]) : kTkBins], 1u);
    __syncthreads();
    if (wave == 0) crossing_2048(s_hist, keff, s_misc);
    __syncthreads();
    const int b1 = (int)s_misc[0];
    uint32_t need = keff - s_misc[1];
    uint32_t cand = s_misc[2];
    uint32_t cm = 0;                 // the thread's keys in bin b1
#pragma unroll
    for (int k = 0; k < kPer; ++k) cm |= (uint32_t)(key[k] != 0 && lbin(key[k]) == b1) << k;
    if (cand > (uint32_t)kRankCap) {
      // Rare (a large crossing bin, e.g. many equal scores): radix digits
      // over the candidates' own key range narrow them.  This path re-reads
      // its keys from memory so that it adds no registers to the common one.
      auto kget = [&](int k) -> uint32_t {
        const int slot = tid * kPer + k;
        return (cm >> k & 1u) ? ks[slot] : 0u;
      };
      for (int i = tid; i < kTkBins; i += kTkThreads) s_hist[i] = 0;
      uint32_t clo = 0xFFFFFFFFu, chi = 0;
#pragma unroll 1
      for (int k = 0; k < kPer; ++k) {
        const uint32_t x = kget(k);
        clo = min(clo, x != 0 ? x : 0xFFFFFFFFu);
        chi = max(chi, x);
      }
      clo = wave_reduce_u32(clo, [](uint32_t x, uint32_t y) { return min(x, y); });
      chi = wave_reduce_u32(chi, [](uint32_t x, uint32_t y) { return max(x, y); });
      if (lane == 0) { s_red[kTkWaves + wave] = clo; s_red[2 * kTkWaves + wave] = chi; }
      __syncthreads();
      clo = 0xFFFFFFFFu; chi = 0;
#pragma unroll 1
      for (int w = 0; w < kTkWaves; ++w) {
        clo = min(clo, s_red[kTkWaves + w]);
        chi = max(chi, s_red[2 * kTkWaves + w]);
      }
      int fixed_lo = highest_diff_bit(clo, chi) + 1;   // bits >= fixed_lo are decided
      uint32_t prefix = (uint32_t)(((uint64_t)clo >> fixed_lo) << fixed_lo);
      while (cand > (uint32_t)kRankCap && fixed_lo > 0) {
        const int sh = max(0, fixed_lo - 11);
        const uint32_t dmask = (1u << (fixed_lo - sh)) - 1;
#pragma unroll 1
        for (int k = 0; k < kPer; ++k) {
          const uint32_t x = kget(k);
          if (x != 0) atomicAdd(&s_hist[(x >> sh) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) crossing_2048(s_hist, need, s_misc);
        __syncthreads();
        prefix |= s_misc[0] << sh;
        need -= s_misc[1];
        cand = s_misc[2];
        fixed_lo = sh;
#pragma unroll 1
        for (int k = 0; k < kPer; ++k) {
          const uint32_t x = kget(k);
          if (x != 0 && ((uint64_t)x >> fixed_lo) != ((uint64_t)prefix >> fixed_lo)) cm &= ~(1u << k);
        }
        for (int i = tid; i < kTkBins; i += kTkThreads) s_hist[i] = 0;   // for a next digit
        __syncthreads();
      }
      if (cand > (uint32_t)kRankCap) {
        T = (int64_t)prefix;           // all bits fixed: a long run of equal keys
        need_eq = need;
        by_scan = true;
      }
    }
    if (!by_scan) {
      // rank the candidates exactly: (key, ~slot) compared as one 64-bit value
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if (cm >> k & 1u) {
          const uint32_t idx = atomicAdd(&s_misc[3], 1u);
          s_cand[idx] = ((uint64_t)key[k] << 32) | (uint32_t)~(uint32_t)(tid * kPer + k);
        }
      }
      __syncthreads();
      for (uint32_t i = tid; i < cand; i += kTkThreads) {
        const uint64_t ci = s_cand[i];
        uint32_t r = 0;
#pragma unroll 8
        for (uint32_t j = 0; j < cand; ++j) r += s_cand[j] > ci;
        if (r == need - 1) { s_misc[0] = (uint32_t)(ci >> 32); s_misc[1] = ~(uint32_t)ci; }
      }
      __syncthreads();
      T = (int64_t)s_misc[0];
      ST = (int)s_misc[1];
    }
  }

  // ordered compaction
  uint32_t eq_before = 0;
  if (by_scan) {
    uint32_t eq = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) eq += key[k] != 0 && (int64_t)key[k] == T;
    eq_before = block_exclusive_scan<kTkThreads>(eq, s_scan, &total);
  }
  uint32_t take = 0, flags = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int slot = tid * kPer + k;
    bool sel = key[k] != 0 && ((int64_t)key[k] > T || ((int64_t)key[k] == T && slot <= ST));
    if (by_scan) {
      const bool eqk = key[k] != 0 && (int64_t)key[k] == T && eq_before < need_eq;
      sel = sel || eqk;
      eq_before += eqk;
    }
    flags |= (uint32_t)sel << k;
    take += sel;
  }
  if (keff == 0) { flags = 0; take = 0; }
  uint32_t before = block_exclusive_scan<kTkThreads>(take, s_scan, &total);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (flags >> k & 1u) {
      if (before < (uint32_t)K) {
        out[before] = blk[k >> 3] * kBlock + (k & 7);
        if (out_s) out_s[before] = key_float(key[k]);
      }
      ++before;
    }
  }
  for (int t = (int)keff + tid; t < K; t += kTkThreads) {
    out[t] = -1;
    if (out_s) out_s[t] = 0.0f;
  }
  if (tid == 0) a.topk_count[q] = (int32_t)keff;
}

template <int D>
hipError_t launch_score(const ReindexArgs& a, hipStream_t s) {
  const int ht = (a.hi + 15) / 16;
  const dim3 grid((unsigned)(a.n_q * a.split)), block(256);
  switch (ht) {
    case 1: hipLaunchKernelGGL((k_reindex_score<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_reindex_score<D, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_reindex_score<D, 3>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_reindex_score<D, 4>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reindex(const ReindexArgs& a, hipStream_t s) {
  hipError_t e = a.d == 64 ? launch_score<64>(a, s) : launch_score<128>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk_select, dim3(a.n_q), dim3(kTkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
