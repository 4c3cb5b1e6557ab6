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
//  * k_reindex_score: split x n_q workgroups; a wave step scores two pool
//    blocks (16 positions, two contiguous 1 KiB key runs at d = 128) with the
//    same f16-MFMA contraction as the Full scan and writes fp32 scores;
//  * k_topk_select: one 1024-thread workgroup per query holds the <= 16,384
//    order-preserving keys in LDS, finds the K-th largest with a radix select
//    that starts at the highest bit where the smallest and largest key differ
//    (the common leading bits would pile every key onto one counter), and
//    compacts in pool order (= ascending positions), admitting keys equal to
//    the threshold lowest position first.
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace csa2 {
namespace {

template <int D, int HT>
__global__ __launch_bounds__(256) void k_reindex_score(ReindexArgs a) {
  constexpr int KC = D / 32;
  constexpr int LB = D / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;
  const int q = blockIdx.x / a.split, part = blockIdx.x % a.split;
  const int cnt = a.pool_count[q];
  const int per = ((a.pool + a.split - 1) / a.split + 1) & ~1;   // even: 2 blocks per step
  const int i_begin = part * per;
  const int i_end = min(cnt, i_begin + per);
  if (i_begin >= i_end) return;
  const int nsteps = (i_end - i_begin + 1) >> 1;
  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);

  v8h qf[HT][KC];
  float wv[HT][4];
  const uint8_t* qp = a.idx_q + (int64_t)q * a.hi * D;
  // all loads issued back to back from clamped (valid) rows, padded heads
  // zeroed afterwards: no branch, one wait
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
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.idx_k + a.seq_base[q] * D, (uint32_t)c * D);
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;
  float* sc = a.scores + (int64_t)q * a.pool * kBlock;

  auto load = [&](int s, uint32_t* kb, int* pos_out) {
    const int i = i_begin + 2 * s + (col >> 3);
    int pos = c;                                   // past the end: reads zero
    if (i < i_end) pos = pool[i] * kBlock + (col & 7);
    if (pos > c || pos < 0) pos = c;
    *pos_out = pos;
    const uint32_t off = (uint32_t)pos * D + gq * LB;
    v4u x = buf_load16(rk, off);
    kb[0] = x[0]; kb[1] = x[1]; kb[2] = x[2]; kb[3] = x[3];
    if constexpr (LB == 32) {
      v4u y = buf_load16(rk, off + 16);
      kb[4] = y[0]; kb[5] = y[1]; kb[6] = y[2]; kb[7] = y[3];
    }
  };

  uint32_t kb[LB / 4];
  int pos = 0;
  if (wave < nsteps) load(wave, kb, &pos);
  for (int s = wave; s < nsteps; s += 4) {
    uint32_t nx[LB / 4];
    int npos = 0;
    const bool more = s + 4 < nsteps;
    if (more) load(s + 4, nx, &npos);
    v8h kf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kf[kc] = fp8x8_to_v8h(kb[2 * kc], kb[2 * kc + 1]);
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
    const int i = i_begin + 2 * s + (col >> 3);
    if (gq == 0 && i < i_end) sc[i * kBlock + (col & 7)] = pos < c ? sum : -__builtin_inff();
    if (more) {
#pragma unroll
      for (int k = 0; k < LB / 4; ++k) kb[k] = nx[k];
      pos = npos;
    }
  }
}

constexpr int kTkThreads = 1024;
constexpr int kMaxCand = 2048 * kBlock;
constexpr int kPer = kMaxCand / kTkThreads;        // 16 items per thread

// LDS slot of item i: one pad word per 16 so that a thread's contiguous run
// and the strided (coalesced) load pattern are both free of bank conflicts.
__device__ __forceinline__ int kslot(int i) { return i + (i >> 4); }

__global__ __launch_bounds__(kTkThreads) void k_topk_select(ReindexArgs a) {
  __shared__ uint32_t s_key[kMaxCand + kMaxCand / 16];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_scan[kTkThreads / 64 + 1];
  __shared__ uint32_t s_misc[4];

  const int q = blockIdx.x, tid = threadIdx.x;
  const int cnt = a.pool_count[q];
  const int N = cnt * kBlock;
  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);
  const int K = a.topk;
  const int32_t* pool = a.pool_blocks + (int64_t)q * a.pool;
  const float* sc = a.scores + (int64_t)q * a.pool * kBlock;
  int32_t* out = a.topk_pos + (int64_t)q * K;
  float* out_s = a.topk_scores ? a.topk_scores + (int64_t)q * K : nullptr;

  // keys in pool order (= ascending positions), coalesced loads; invalid -> 0
  uint32_t nvalid = 0, lo = 0xFFFFFFFFu, hi = 0;
  for (int k = 0; k < kPer; ++k) {
    const int i = k * kTkThreads + tid;
    uint32_t key = 0;
    if (i < N) {
      const int pos = pool[i >> 3] * kBlock + (i & 7);
      if (pos >= 0 && pos < c) {
        key = order_key(sc[i]);
        ++nvalid;
        lo = min(lo, key);
        hi = max(hi, key);
      }
    }
    s_key[kslot(i)] = key;
  }
  uint32_t total;
  (void)block_exclusive_scan<kTkThreads>(nvalid, s_scan, &total);
  const uint32_t keff = min((uint32_t)K, total);
  const uint32_t kmin = block_min_u32<kTkThreads>(lo, s_scan);
  const uint32_t kmax = block_max_u32<kTkThreads>(hi, s_scan);

  uint32_t T = 0, need_eq = 0;
  if (keff > 0) {
    const int top = highest_diff_bit(kmin, kmax);
    uint32_t prefix = (uint32_t)(((uint64_t)kmin >> (top + 1)) << (top + 1));
    uint32_t need = keff;
    int fixed_lo = top + 1;            // bits >= fixed_lo are decided
    while (fixed_lo > 0) {
      const int sh = max(0, fixed_lo - 8);
      const uint32_t dmask = (1u << (fixed_lo - sh)) - 1;
      if (tid < 256) s_hist[tid] = 0;
      __syncthreads();
      for (int k = 0; k < kPer; ++k) {
        const uint32_t key = s_key[kslot(tid * kPer + k)];
        if (key != 0 && ((uint64_t)key >> fixed_lo) == ((uint64_t)prefix >> fixed_lo))
          atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
      }
      __syncthreads();
      find_crossing(s_hist, 256, need, s_misc);
      __syncthreads();
      prefix |= s_misc[0] << sh;
      need -= s_misc[1];
      fixed_lo = sh;
      __syncthreads();
    }
    T = prefix;
    need_eq = need;
  }

  // ordered compaction: key > T always, key == T lowest positions first
  uint32_t eq = 0;
  if (keff > 0) {
    for (int k = 0; k < kPer; ++k) eq += s_key[kslot(tid * kPer + k)] == T;
  }
  uint32_t eq_before = block_exclusive_scan<kTkThreads>(eq, s_scan, &total);
  uint32_t take = 0;
  uint32_t flags = 0;
  if (keff > 0) {
    for (int k = 0; k < kPer; ++k) {
      const uint32_t key = s_key[kslot(tid * kPer + k)];
      bool sel = key > T;
      if (key == T && eq_before < need_eq) { sel = true; ++eq_before; }
      if (sel) { flags |= 1u << k; ++take; }
    }
  }
  uint32_t before = block_exclusive_scan<kTkThreads>(take, s_scan, &total);
  for (int k = 0; k < kPer; ++k) {
    if (flags & (1u << k)) {
      const int i = tid * kPer + k;
      if (before < (uint32_t)K) {
        out[before] = pool[i >> 3] * kBlock + (i & 7);
        if (out_s) out_s[before] = key_float(s_key[kslot(i)]);
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
