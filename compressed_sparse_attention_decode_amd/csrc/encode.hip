// FP4 main-KV encode: E2M1 codes with one E4M3 scale per 16 latent channels.
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (FP4 main KV: E2M1 with one E4M3
// scale per 16 channels) and the FP4Quantizer of section 8 of the newsaint.id
// page "DeepSeek-V4.1-Flash 2026: Arsitektur ... CSA2, FP4 KV Caching ..."
// (scale = group amax / 6 clamped to 448, nearest E2M1 level).  The scale is
// rounded to E4M3 with round-to-nearest-even, E2M1 ties go to the even code.
//
// One thread per 16-channel group: 32 bytes of bf16 in, 8 code bytes and one
// scale byte out.  A 256-thread block covers 8 entries; the bf16 reads and the
// code writes are contiguous across the block.  HBM-bound (1,576 bytes moved
// per entry, about 4 ALU ops per byte).
//
// k_encode_rows applies the same per-group codec to rows of any power-of-two
// multiple of 16 channels with no RoPE part: the FP4 indexer rows (§4 of the
// newsaint.id page: DeepSeek-V4 trained the indexer's query and key with FP4
// QAT) are 128-channel rows of this format.
//
// Group-32 variant of the main-KV codec (the akhunji.com page, "Microscopic
// FP4 (E2M1) Cache Compression": block-level FP8 scaling over blocks of 32
// elements): the same scale rule and E2M1 rounding over 32-channel groups,
// one thread per group, 16 scale bytes per entry.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

// RNE of t in [0, 448] to an E4M3FN code (0x00..0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  if (t < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);   // 8 -> 0x08 = 2^-6, still right
  }
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);          // round mantissa to 3 bits, ties to even
  return (u >> 20) - (120u << 3);
}

// One group of G = 16 or 32 channels (2G bytes of bf16 at `src`): its G / 8
// code dwords (channel 8j + i in nibble i of dword j) and its scale byte as
// the return value.
template <int G>
__device__ __forceinline__ uint32_t encode_group(const uint16_t* src, uint32_t (&packed)[G / 8]) {
  uint32_t w[G / 2];
  const v4u* s16 = reinterpret_cast<const v4u*>(src);
#pragma unroll
  for (int j = 0; j < G / 8; ++j) {
    const v4u a = s16[j];
    w[4 * j + 0] = a[0]; w[4 * j + 1] = a[1]; w[4 * j + 2] = a[2]; w[4 * j + 3] = a[3];
  }

  // group maximum of |x| on the bit patterns (finite bf16 magnitudes order as integers)
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < G / 2; ++i) {
    amax = max(amax, w[i] & 0x7FFFu);
    amax = max(amax, (w[i] >> 16) & 0x7FFFu);
  }
  const float t = fminf(__uint_as_float(amax << 16) / 6.0f, 448.0f);
  const uint32_t S = e4m3_rne(t);
  const float s = e4m3_to_float(S);

#pragma unroll
  for (int j = 0; j < G / 8; ++j) packed[j] = 0;
  if (s != 0.0f) {
    const float t025 = 0.25f * s, t075 = 0.75f * s, t125 = 1.25f * s, t175 = 1.75f * s;
    const float t250 = 2.5f * s, t350 = 3.5f * s, t500 = 5.0f * s;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint32_t bits = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const float ax = __uint_as_float((bits & 0x7FFFu) << 16);
      // nearest E2M1 level, ties to the even code: strict at ties whose lower
      // neighbour is even, inclusive where the upper neighbour is even.
      uint32_t m = (ax > t025) + (ax >= t075) + (ax > t125) + (ax >= t175) +
                   (ax > t250) + (ax >= t350) + (ax > t500);
      const uint32_t code = ((bits >> 12) & 8u) | m;
      packed[i >> 3] |= code << (4 * (i & 7));
    }
  }
  return S;
}

// Main-KV entries, G-channel groups: 512 / G threads per entry.
template <int G>
__global__ __launch_bounds__(256) void k_encode(int64_t n, const uint16_t* __restrict__ latent,
                                                const uint16_t* __restrict__ rope,
                                                const int64_t* __restrict__ dst_row,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                uint16_t* __restrict__ rope_out) {
  constexpr int NG = kLatent / G;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = gid / NG;
  const int g = (int)(gid % NG);
  if (e >= n) return;
  const int64_t row = dst_row ? dst_row[e] : e;
  uint32_t packed[G / 8];
  const uint32_t S = encode_group<G>(latent + e * kLatent + g * G, packed);
  if constexpr (G == 16) {
    *reinterpret_cast<v2u*>(codes + row * kCodeBytes + g * 8) = v2u{packed[0], packed[1]};
  } else {
    *reinterpret_cast<v4u*>(codes + row * kCodeBytes + g * 16) = v4u{packed[0], packed[1], packed[2], packed[3]};
  }
  scales[row * NG + g] = (uint8_t)S;
  if (g < 8) {
    const v4u* rs = reinterpret_cast<const v4u*>(rope + e * kRope + g * 8);
    *reinterpret_cast<v4u*>(rope_out + row * kRope + g * 8) = rs[0];
  }
}

// Rows of 16 << lg channels: one thread per group, 1 << lg groups per row.
__global__ __launch_bounds__(256) void k_encode_rows(int64_t n, int lg, const uint16_t* __restrict__ src,
                                                     const int64_t* __restrict__ dst_row,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = gid >> lg;
  const int g = (int)(gid & ((1 << lg) - 1));
  if (e >= n) return;
  const int64_t row = dst_row ? dst_row[e] : e;
  const int64_t groups = (int64_t)1 << lg;
  uint32_t packed[2];
  const uint32_t S = encode_group<kGroup>(src + (e * groups + g) * kGroup, packed);
  *reinterpret_cast<v2u*>(codes + (row * groups + g) * 8) = v2u{packed[0], packed[1]};
  scales[row * groups + g] = (uint8_t)S;
}

// Rows of (sequence, position) pairs in paged planes: entry i is position
// pos[i] of the sequence whose page-table row starts at table_off[i].
__global__ __launch_bounds__(256) void k_page_rows(int64_t n, const int32_t* pages, int shift,
                                                   const int64_t* table_off, const int32_t* pos, int64_t* dst_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t p = pos[i];
  const int64_t page = pages[table_off[i] + (p >> shift)];
  dst_row[i] = (page << shift) | (p & ((1 << shift) - 1));
}

}  // namespace

hipError_t launch_page_rows(int64_t n, const int32_t* pages, int page_shift, const int64_t* table_off,
                            const int32_t* pos, int64_t* dst_row, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_page_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, pages, page_shift,
                     table_off, pos, dst_row);
  return hipGetLastError();
}

hipError_t launch_encode_rows(int64_t n, int width, const uint16_t* src, const int64_t* dst_row,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int lg = 0;
  while ((kGroup << lg) < width) ++lg;
  if ((kGroup << lg) != width) return hipErrorInvalidValue;
  const int64_t blocks = ((n << lg) + 255) / 256;
  hipLaunchKernelGGL(k_encode_rows, dim3((unsigned)blocks), dim3(256), 0, s, n, lg, src, dst_row, codes, scales);
  return hipGetLastError();
}

hipError_t launch_encode(int64_t n, int group, const uint16_t* latent, const uint16_t* rope,
                         const int64_t* dst_row, uint8_t* codes, uint8_t* scales,
                         uint16_t* rope_out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (group != 16 && group != 32) return hipErrorInvalidValue;
  const int64_t threads = n * (kLatent / group);
  const int64_t blocks = (threads + 255) / 256;
  if (group == 16)
    hipLaunchKernelGGL(k_encode<16>, dim3((unsigned)blocks), dim3(256), 0, s, n, latent, rope, dst_row,
                       codes, scales, rope_out);
  else
    hipLaunchKernelGGL(k_encode<32>, dim3((unsigned)blocks), dim3(256), 0, s, n, latent, rope, dst_row,
                       codes, scales, rope_out);
  return hipGetLastError();
}

}  // namespace csa2
