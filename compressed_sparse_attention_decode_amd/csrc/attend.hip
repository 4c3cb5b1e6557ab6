// Core attention over the kept FP4 entries and the bf16 sliding window, with
// one softmax and a 512-wide latent output per head (MLA-absorbed).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (heterogeneous KV: the same main Q
// attends the sparse main-KV branch and the uncompressed window branch and
// the two are merged; mode table: Reuse layers change only Q) and §4 of the
// newsaint.id page (FP4 main KV dequantised just before attention).  The key
// of a sparse entry is [dequantised latent (512) || bf16 rope (64)] and its
// value is the dequantised latent; a window row supplies both from bf16.
//
// Mapping (gfx950): a workgroup = one query x up to 64 heads (one wave per 16
// heads) x one split of the entry list.  Entries stream in tiles of 32:
//  * the workgroup gathers the tile's rows (FP4 codes + E4M3 scales + rope,
//    or window rows), dequantises on load (exact in bf16 and f16) and stores
//    two LDS images: keys row-major in bf16 (for Q.K) and values transposed
//    in f16 (for P.V);
//  * Q.K^T: v_mfma_f32_16x16x32_bf16 with the tile as A (rows = entries) and
//    the wave's 16 query heads as B (held in registers), giving S^T whose lane
//    layout is exactly the A layout P.V needs, so P never leaves registers;
//  * online softmax in the exp2 domain, P rounded to f16 (bf16 would cost
//    about 2^-9 relative per weight), P.V with v_mfma_f32_16x16x32_f16 into
//    32 accumulator tiles (16 heads x 512 dims);
//  * with several splits per query, unnormalised partials (o, m, l) are
//    merged by k_attend_combine with a log-sum-exp rescale.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kTile = kAttendTile;        // 32 entries
constexpr int kKLS = kKeyDim + 8;         // bf16 row stride of the key image
constexpr int kVTS = kTile + 4;           // f16 row stride of the value image

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  const uint32_t m = nib & 7u;
  float v = m < 2 ? 0.5f * (float)m : __uint_as_float((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
  return (nib & 8u) ? -v : v;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_attend(AttendArgs a) {
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kTile * kKLS];     // bf16 keys
  __shared__ __attribute__((aligned(16))) _Float16 s_v[kLatent * kVTS];   // f16 values^T

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;
  const int S = a.splits, HG = a.head_groups;
  const int q = blockIdx.x / (HG * S);
  const int hg = (blockIdx.x / S) % HG;
  const int sp = blockIdx.x % S;
  const int H = a.heads;
  const int head0 = (hg * NW + wave) * 16;

  const int n = a.n_visible[q];
  const int c = max(0, n - a.swa);
  const int Es = min(a.topk_count[q], a.topk);
  const int E = Es + (n - c);
  const int e_begin = sp * a.split_entries;
  const int e_end = min(E, e_begin + a.split_entries);
  const int64_t seq_base = a.seq_base[q];
  const int64_t swa_base = a.swa_base[q];
  const int32_t* tk = a.topk_pos + (int64_t)q * a.topk;

  // query fragments: B operand, lane = head (col), k-slots = dims 32ks + 8gq + j
  v8bf qf[kKeyDim / 32];
  {
    const int h = head0 + col;
#pragma unroll
    for (int ks = 0; ks < kKeyDim / 32; ++ks) {
      const int d = ks * 32 + gq * 8;
      const uint16_t* src = d < kLatent ? a.q_lat + ((int64_t)q * H + h) * kLatent + d
                                        : a.q_rope + ((int64_t)q * H + h) * kRope + (d - kLatent);
      v4u raw = *reinterpret_cast<const v4u*>(src);
      qf[ks] = __builtin_bit_cast(v8bf, raw);
    }
  }

  float m = -__builtin_inff(), l = 0.0f;
  v4f o[kLatent / 16];
#pragma unroll
  for (int nt = 0; nt < kLatent / 16; ++nt) o[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int e0 = e_begin; e0 < e_end; e0 += kTile) {
    const int ne = min(kTile, e_end - e0);
    __syncthreads();
    // ---- gather + dequantise the tile into LDS
    for (int it = tid; it < kTile * 32; it += NT) {
      const int e = it >> 5, grp = it & 31, ge = e0 + e;
      uint32_t kw[8] = {0, 0, 0, 0, 0, 0, 0, 0};     // 16 bf16
      _Float16 vh[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) vh[k] = (_Float16)0.0f;
      if (e < ne) {
        if (ge < Es) {
          const int64_t row = seq_base + tk[ge];
          const v2u cw = *reinterpret_cast<const v2u*>(a.kv_codes + row * kCodeBytes + grp * 8);
          const float s = e4m3_to_float(a.kv_scales[row * kScaleBytes + grp]);
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const uint32_t nib = (cw[k >> 3] >> (4 * (k & 7))) & 15u;
            const float v = e2m1_value(nib) * s;            // exact
            vh[k] = (_Float16)v;
            kw[k >> 1] |= (__float_as_uint(v) >> 16) << (16 * (k & 1));
          }
        } else {
          const int64_t row = swa_base + (ge - Es);
          const v4u* src = reinterpret_cast<const v4u*>(a.swa_kv + row * kKeyDim + grp * 16);
          const v4u x0 = src[0], x1 = src[1];
          kw[0] = x0[0]; kw[1] = x0[1]; kw[2] = x0[2]; kw[3] = x0[3];
          kw[4] = x1[0]; kw[5] = x1[1]; kw[6] = x1[2]; kw[7] = x1[3];
#pragma unroll
          for (int k = 0; k < 16; ++k) vh[k] = (_Float16)bf16_to_float((kw[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
        }
      }
      v4u* dk = reinterpret_cast<v4u*>(s_k + e * kKLS + grp * 16);
      dk[0] = v4u{kw[0], kw[1], kw[2], kw[3]};
      dk[1] = v4u{kw[4], kw[5], kw[6], kw[7]};
#pragma unroll
      for (int k = 0; k < 16; ++k) s_v[(grp * 16 + k) * kVTS + e] = vh[k];
    }
    for (int it = tid; it < kTile * 8; it += NT) {
      const int e = it >> 3, ch = it & 7, ge = e0 + e;
      v4u x = {0, 0, 0, 0};
      if (e < ne) {
        if (ge < Es) x = *reinterpret_cast<const v4u*>(a.kv_rope + (seq_base + tk[ge]) * kRope + ch * 8);
        else x = *reinterpret_cast<const v4u*>(a.swa_kv + (swa_base + (ge - Es)) * kKeyDim + kLatent + ch * 8);
      }
      *reinterpret_cast<v4u*>(s_k + e * kKLS + kLatent + ch * 8) = x;
    }
    __syncthreads();
    if (head0 >= H) continue;

    // ---- S^T = K_tile . Q^T  (rows: entries, cols: heads)
    v4f s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kKeyDim / 32; ++ks) {
      const v8bf k0 = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(s_k + col * kKLS + ks * 32 + gq * 8));
      const v8bf k1 = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(s_k + (16 + col) * kKLS + ks * 32 + gq * 8));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
    // lane holds entries 4gq+i (s0) and 16+4gq+i (s1) for head `col`
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (4 * gq + i < ne) ? s0[i] * a.scale_log2 : -__builtin_inff();
      sv[4 + i] = (16 + 4 * gq + i < ne) ? s1[i] * a.scale_log2 : -__builtin_inff();
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m, mt);                 // finite: the tile has an entry
    const float alpha = exp2f(m - m_new);
    v8h pf;
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = exp2f(sv[i] - m_new);
      ls += p;
      pf[i] = (_Float16)p;
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l = l * alpha + ls;
    m = m_new;
    // rescale accumulator rows (heads 4gq+i) by their alpha
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * gq + i, 64);
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= ar[i];
    }
    // ---- O += P . V  (A = P: rows heads, k = entries {4gq..4gq+3, 16+4gq..+3})
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt) {
      const _Float16* vr = s_v + (nt * 16 + col) * kVTS;
      const v2u lo = *reinterpret_cast<const v2u*>(vr + 4 * gq);
      const v2u hi = *reinterpret_cast<const v2u*>(vr + 16 + 4 * gq);
      const v8h vb = __builtin_bit_cast(v8h, v4u{lo[0], lo[1], hi[0], hi[1]});
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vb, o[nt], 0, 0, 0);
    }
  }
  if (head0 >= H) return;

  // ---- epilogue: lane holds O[head 4gq+i][dim 16nt+col]
  if (S == 1) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l, 4 * gq + i, 64);
      inv[i] = li > 0.0f ? 1.0f / li : 0.0f;
    }
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.out[((int64_t)q * H + head0 + 4 * gq + i) * kLatent + nt * 16 + col] = o[nt][i] * inv[i];
    }
    if (a.lse && gq == 0)
      a.lse[(int64_t)q * H + head0 + col] = l > 0.0f ? (m + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
  } else {
    float* po = a.part_o + (((int64_t)q * S + sp) * H + head0) * kLatent;
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(4 * gq + i) * kLatent + nt * 16 + col] = o[nt][i];
    }
    if (gq == 0) {
      float* pm = a.part_ml + (((int64_t)q * S + sp) * H + head0 + col) * 2;
      pm[0] = m;
      pm[1] = l;
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void k_attend_combine(AttendArgs a) {
  const int q = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
  const int S = a.splits, H = a.heads;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[(((int64_t)q * S + s) * H + h) * 2]);
  float den = 0.0f;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int d0 = threadIdx.x * 4;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float* pm = a.part_ml + (((int64_t)q * S + s) * H + h) * 2;
      if (pm[1] == 0.0f) continue;
      const float wgt = exp2f(pm[0] - M);
      den += wgt * pm[1];
      const v4f ov = *reinterpret_cast<const v4f*>(a.part_o + (((int64_t)q * S + s) * H + h) * kLatent + d0);
      for (int k = 0; k < 4; ++k) acc[k] += wgt * ov[k];
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  *reinterpret_cast<v4f*>(a.out + ((int64_t)q * H + h) * kLatent + d0) =
      v4f{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)q * H + h] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
}

template <int NW>
hipError_t launch_nw(const AttendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_q * a.head_groups * a.splits)), block(64 * NW);
  hipLaunchKernelGGL((k_attend<NW>), grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(k_attend_combine, dim3((unsigned)(a.n_q * a.heads)), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attend_waves(int heads) {
  const int t = heads / 16;
  return t % 4 == 0 ? 4 : (t % 2 == 0 ? 2 : 1);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  switch (a.heads / a.head_groups / 16) {
    case 4: return launch_nw<4>(a, s);
    case 2: return launch_nw<2>(a, s);
    default: return launch_nw<1>(a, s);
  }
}

}  // namespace csa2
