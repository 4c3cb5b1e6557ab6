// Full-mode indexer scan: per-position scores, block-of-8 maxima and a
// coarse histogram of the block scores.
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (hierarchical sparse indexer: the
// first Full layer scores the whole visible context and pools blocks of 8;
// mode table: Full runs the indexer over every position) and §3 of the
// newsaint.id page (the Full-mode indexer must scan every causally visible
// position, O(N)).  Score of position p (the pages give no formula; reading
// used throughout this library): s_p = sum_h w_h * max(0, q_h . k_p).
//
// Layout and mapping (gfx950):
//  * one workgroup = 4 waves = one query x kScanTile consecutive positions;
//  * a wave step covers 16 positions: lane l holds key row (l & 15) and the
//    contiguous byte range [(l >> 4) * d/4, +d/4) of that row, loaded with raw
//    buffer loads (rows >= c read as zero, so the tail needs no branches);
//  * fp8 keys and queries are converted to f16 in registers (exact) and
//    contracted with v_mfma_f32_16x16x32_f16: A = 16 query heads, B = 16
//    positions, K = 32 dims per instruction.  The product and the fp32
//    accumulation are exact for fp8 inputs; the fp8 MFMA is not (its
//    accumulator drops low-order bits), so it is not used;
//  * the epilogue applies ReLU and the head weights, reduces over the four
//    lane groups, masks p >= c, takes the max over 8 lanes (one block), and
//    one lane per block writes the block score and bumps an LDS histogram of
//    the top 12 key bits, flushed once per workgroup with global atomics.
// HBM-bound: 128 bytes of keys per position, 16 KFLOP per position.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

template <int D, int HT>
__global__ __launch_bounds__(256) void k_scan(ScanArgs a) {
  constexpr int KC = D / 32;            // MFMA k-chunks
  constexpr int LB = D / 4;             // bytes per lane per position row
  __shared__ uint32_t s_hist[kHistBins];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;

  // block -> (query, tile); the g tokens of one sequence and the same tile
  // land on the same XCD (block ids equal mod 8) so their key reads share L2.
  const int g = a.g;
  const int bid = blockIdx.x;
  const int unit = (bid / (8 * g)) * 8 + (bid & 7);
  const int j = (bid >> 3) % g;
  const int n_groups = a.n_q / g;
  const int group = unit % n_groups, tile = unit / n_groups;
  if (tile >= a.tiles) return;
  const int q = group * g + j;

  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);
  const int p_begin = tile * kScanTile;
  if (p_begin >= c) return;
  const int p_end = min(p_begin + kScanTile, c);
  const int nsteps = (p_end - p_begin + 15) >> 4;

  for (int i = tid; i < kHistBins; i += 256) s_hist[i] = 0;

  // query fragments (f16) and head weights for this lane
  v8h qf[HT][KC];
  float wv[HT][4];
  const uint8_t* qp = a.idx_q + (int64_t)q * a.hi * D;
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int h = t * 16 + col;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint32_t w0 = 0, w1 = 0;
      if (h < a.hi) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(qp + (int64_t)h * D + gq * LB + kc * 8);
        w0 = src[0];
        w1 = src[1];
      }
      qf[t][kc] = fp8x8_to_v8h(w0, w1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = t * 16 + gq * 4 + i;
      wv[t][i] = hh < a.hi ? a.idx_w[(int64_t)q * a.hi + hh] : 0.0f;
    }
  }

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.idx_k + a.seq_base[q] * D, (uint32_t)c * D);
  float* bs = a.bscore + (int64_t)q * a.ld;
  __syncthreads();

  auto load = [&](int s, uint32_t* kb) {
    const uint32_t off = (uint32_t)(p_begin + s * 16 + col) * D + gq * LB;
    v4u x = buf_load16(rk, off);
    kb[0] = x[0]; kb[1] = x[1]; kb[2] = x[2]; kb[3] = x[3];
    if constexpr (LB == 32) {
      v4u y = buf_load16(rk, off + 16);
      kb[4] = y[0]; kb[5] = y[1]; kb[6] = y[2]; kb[7] = y[3];
    }
  };

  uint32_t kb[LB / 4];
  if (wave < nsteps) load(wave, kb);
  for (int s = wave; s < nsteps; s += 4) {
    uint32_t nx[LB / 4];
    const bool more = s + 4 < nsteps;
    if (more) load(s + 4, nx);

    v8h kf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kf[kc] = fp8x8_to_v8h(kb[2 * kc], kb[2 * kc + 1]);
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[t][kc], kf[kc], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wv[t][i] * fmaxf(acc[i], 0.0f);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    const int p0 = p_begin + s * 16;
    float v = (p0 + col < c) ? part : -__builtin_inff();
    v = fmaxf(v, __shfl_xor(v, 1, 64));
    v = fmaxf(v, __shfl_xor(v, 2, 64));
    v = fmaxf(v, __shfl_xor(v, 4, 64));
    if (lane < 16 && (lane & 7) == 0) {
      const int jb = (p0 + lane) >> 3;
      if (jb * 8 < c) {
        bs[jb] = v;
        atomicAdd(&s_hist[order_key(v) >> kHistShift], 1u);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < LB / 4; ++i) kb[i] = nx[i];
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)q * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) {
    const uint32_t v = s_hist[i];
    if (v) atomicAdd(gh + i, v);
  }
}

template <int D>
hipError_t launch_d(const ScanArgs& a, hipStream_t s) {
  const int ht = (a.hi + 15) / 16;
  const int units = ((a.n_q / a.g) * a.tiles + 7) / 8 * 8;
  const dim3 grid((unsigned)(units * a.g)), block(256);
  switch (ht) {
    case 1: hipLaunchKernelGGL((k_scan<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_scan<D, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_scan<D, 3>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_scan<D, 4>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.tiles == 0) return hipSuccess;
  return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace csa2
