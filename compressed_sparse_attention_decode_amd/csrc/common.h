// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace csa2 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kLatent = 512;           // latent width shared across heads
constexpr int kRope = 64;              // bf16 RoPE key width
constexpr int kKeyDim = kLatent + kRope;
constexpr int kGroup = 16;             // channels per E4M3 scale
constexpr int kCodeBytes = kLatent / 2;
constexpr int kScaleBytes = kLatent / kGroup;
constexpr int kBlock = 8;              // indexer block
constexpr int kWave = 64;

// Order-preserving map float -> uint32 (larger float -> larger key); -0 and
// +0 map to the same key so equal scores tie exactly.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// A wave-uniform read of memory that no kernel writes while it runs, through
// the scalar cache: the constant address space lets the compiler use a scalar
// load where it cannot prove on its own that nothing in the kernel clobbers
// the location (a vector load there makes every address built from the value
// divergent, and buffer loads over it waterfall loops).
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v4u buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Four OCP E4M3FN bytes -> four f16 (exact: every E4M3 value is an f16).
__device__ __forceinline__ void fp8x4_to_f16(uint32_t x, _Float16* o) {
  v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// Eight E4M3 bytes (two dwords) -> one v8h MFMA operand.
__device__ __forceinline__ v8h fp8x8_to_v8h(uint32_t a, uint32_t b) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false);
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true);
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// D += A B^T over 128 E4M3 k-slots with unit block scales (gfx950
// v_mfma_scale_f32_16x16x128_f8f6f4, E8M0 scale 127 = 1.0): A row = lane
// & 15, B column = lane & 15, 32 bytes of k-slots per lane; any byte -> k-slot
// map that A and B share gives the same dot products.  The products are exact
// (E4M3 x E4M3); the instruction's internal accumulation keeps fewer bits
// than fp32 (measured: scores within about 3e-5 relative on N(0,1) keys).
__device__ __forceinline__ v4f mfma_fp8_k128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// Two 16-byte halves as one 32-byte MFMA operand.
__device__ __forceinline__ v8i cat_v8i(v4u lo, v4u hi) {
  return __builtin_bit_cast(v8i, (__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
}

// Eight E2M1 codes (one dword, low nibble = lower channel) times their
// group's E4M3 scale, given as f16 in both halves of s2: one v8h MFMA
// operand.  Exact: the gfx950 conversion at scale 1.0 gives the E2M1 level,
// and level x scale needs at most 6 significant bits within [2^-10, 2688].
__device__ __forceinline__ v8h fp4x8_to_v8h(uint32_t w, v2h s2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The two E4M3 scale bytes of a lane's 32 FP4 channels (groups 2*gq and
// 2*gq + 1 of a 128-wide row, whose 8 scale bytes sit in two dwords): `sw`
// is the dword holding them, `hi` selects its upper half.  Returns the two
// scales as f16 (exact).
__device__ __forceinline__ v2h fp4_pair_scales(uint32_t sw, bool hi) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi ? sw >> 16 : sw, 1.0f, false);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// E4M3FN byte -> float (scale decode; NaN codes are not produced by encode).
__device__ __forceinline__ float e4m3_to_float(uint32_t c) {
  uint32_t e = (c >> 3) & 15, m = c & 7;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80) ? -v : v;
}

// Cross-lane reductions without LDS round trips (gfx950).
// Sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48): two
// row swaps.  Every lane ends with the same value, added in the same order.
__device__ __forceinline__ float sum_rows4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of 8 lanes: quad_perm [1,0,3,2], [2,3,0,1],
// then row_half_mirror (lane i <-> 7 - i within each 8).
__device__ __forceinline__ float max_lanes8(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  return fmaxf(v, dpp_mov<0x141>(v));
}

// Reduction over the 64 lanes of a wave without LDS: DPP within each row of
// 16 (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror), then the
// gfx950 row swaps across the four rows.  Every lane ends with the result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r[0], r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave without LDS: DPP row
// shifts by 1, 2, 4 and 8 scan each row of 16 (lanes shifted in from outside
// the row read 0), then row_bcast:15 adds row r's last lane to row r + 1 and
// row_bcast:31 adds lane 31 to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

// Block-wide exclusive scan of one uint32 per thread (blockDim.x = NT, a
// multiple of 64).  `sh` needs NT/64 words.  Returns the exclusive prefix;
// *total receives the block sum.  Each wave scans in registers and publishes
// its sum; every thread then adds the sums of the waves before its own.
// Contains two __syncthreads() (the second lets `sh` be reused at once).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan_u32(v);
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sh[w];
    before += w < wave ? t : 0u;
    sum += t;
  }
  *total = sum;
  __syncthreads();
  return before + x - v;
}

}  // namespace csa2
