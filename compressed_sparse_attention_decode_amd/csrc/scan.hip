// Full-mode indexer scan: per-position scores and block-of-8 maxima.
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (hierarchical sparse indexer: the
// first Full layer scores the whole visible context and pools blocks of 8;
// mode table: Full runs the indexer over every position) and §3 of the
// newsaint.id page (the Full-mode indexer must scan every causally visible
// position, O(N)).  Score of position p (the pages give no formula; reading
// used throughout this library): s_p = sum_h w_h * max(0, q_h . k_p).
//
// Layout and mapping (gfx950):
//  * one workgroup = 4 waves = one query x tile_pos consecutive positions;
//  * a wave step covers 16 positions: lane l holds d/4 bytes of key row
//    (l & 15).  Keys stream with direct-to-LDS raw buffer loads (rows >= c
//    read as zero, so the tail needs no branches) through a ring of R LDS
//    slots per wave, R - 1 steps in flight, which costs no VGPRs.  Each load
//    instruction covers whole 128-byte lines with the nontemporal hint: the
//    keys are read once, and a line split over two instructions would be
//    fetched twice;
//  * fp8 rows: the raw e4m3 bytes go straight into the gfx950 fp8 MFMA,
//    v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (A = 16 query heads,
//    B = 16 positions, K = 128 dims: one instruction per 16 heads and step;
//    d = 64 pads K with zeros), so no conversion runs in the loop.  The
//    products are exact; the instruction's internal accumulation keeps fewer
//    bits than fp32.  Measured against the exact scores: within 3.4e-5
//    relative on N(0,1) e4m3 inputs at 128K and 1M positions (1.1e-4 on
//    wide-range ones), and over 48 queries x 131,072 positions every pool
//    and Top-512 set either matched the exact one or differed only inside
//    the 1e-5 band (largest gap of a differing index 3.8e-6 relative).  The
//    f16 MFMA on exactly converted values (products exact, fp32 sums) stays
//    within 2.4e-7 but needs 16 conversions and 4x the MFMA issues per step;
//  * the epilogue applies ReLU and the head weights, reduces over the four
//    lane groups, masks p >= c, takes the max over 8 lanes (one block), and
//    one lane per block writes the block score to LDS; the tile's scores
//    leave in one coalesced store (4 bytes per 1 KiB of keys).
// HBM-bound: 128 bytes of keys per position, 16 KFLOP per position.
//
// FP4 indexer rows (§4 of the newsaint.id page: DeepSeek-V4 trained the
// indexer's query and key with FP4 QAT), d = 128 only: a key is 64 bytes of
// E2M1 codes plus 8 E4M3 scale bytes (one per 16 channels), the query the
// same per head.  A wave step then moves 1 KiB of codes (lane l: row l & 15,
// channels 32 (l >> 4) .. +32) and the step's 128 scale bytes into the ring;
// codes times scale are exact in f16 and feed v_mfma_f32_16x16x32_f16 (the
// fp8f6f4 MFMA takes power-of-two block scales over 32 values, not E4M3
// scales over 16).  72 bytes per position.
#include "common.h"
#include "scan_args.h"

namespace csa2 {
namespace {

// Byte offset, inside a key row, of the MFMA lane's 16-byte chunk `h` (h = 0,
// 1).  For d = 128 chunk 0 covers bytes [16gq, 16gq+16) and chunk 1 bytes
// [64+16gq, ...).  The query fragments use the same byte -> k-slot map, so the
// permutation of the reduction dimension cancels in every dot product.
template <int D>
__device__ __forceinline__ int key_chunk(int gq, int h) {
  return D == 128 ? h * 64 + gq * 16 : gq * 16;
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]); the fields not named are left at "no wait".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

constexpr int kMaxTilePos = 4096;

constexpr uint32_t kOob = 0xFFFFFF00u;   // a buffer offset past any row: reads zero

template <int D, int HT, int R, int NW, bool F4, bool PG, bool PS>
__global__ __launch_bounds__(64 * NW) void k_scan(ScanArgs a) {
  static_assert(!F4 || D == 128, "FP4 rows are 128 channels wide");
  constexpr int NT = 64 * NW;
  constexpr int KC = D / 32;            // MFMA k-chunks of 32 dims
  constexpr int NH = F4 ? 1 : D / 64;   // 16-byte key loads per lane per step
  constexpr int LPS = F4 ? 2 : NH;      // load instructions per lane per step (FP4: + scales)
  constexpr int RB = F4 ? D / 2 : D;    // key code bytes per position
  constexpr int SB = D / 16;            // FP4 scale bytes per position
  constexpr int SLOT = F4 ? 1024 + 256 : NH * 1024;   // LDS bytes per ring slot
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[NW][R][SLOT];
  __shared__ float s_bs[kMaxTilePos / 8];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[64 * D];
  __shared__ __attribute__((aligned(16))) float s_w[64];
  __shared__ int32_t s_pg[PG ? kMaxTilePos / 16 + 1 : 1];   // paged: the tile's page ids
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, col = lane & 15;

  // block -> (query, tile); the g tokens of one sequence and the same tile
  // land on the same XCD (block ids equal mod 8) so their key reads share L2.
  // Eight sequences or fewer: XCD x takes sequences x, x + 8, ... whole.
  // More: the sequences rotate across tiles (tile t of sequence s is unit
  // t n_groups + (s - t) mod n_groups), so each XCD takes an equal share of
  // every sequence's tiles.  Whole sequences left the XCDs up to 1.46x apart
  // in work on a batch of 32 contexts drawn from [32K, 256K] (the kernel
  // waits for the busiest XCD); for 8 equal sequences the rotation measured
  // 0.6 us slower.
  // One, two or four sequences of single tokens: each sequence's XCDs take
  // contiguous runs of its tiles, a run of long tiles (dispatched first)
  // and a run of short ones, instead of every eighth tile (measured: 0.6 us
  // less for one sequence of 1M positions).
  const int g = a.g;
  const int bid = blockIdx.x;
  const int unit = (bid / (8 * g)) * 8 + (bid & 7);
  const int j = (bid >> 3) % g;
  const int n_groups = a.n_q / g;
  int tile = unit / n_groups, group = unit % n_groups;
  if (n_groups > 8) group = (group + tile) % n_groups;
  if (g == 1 && n_groups < 8 && 8 % n_groups == 0 && a.tiles % (16 / n_groups) == 0) {
    const int X = 8 / n_groups;                   // XCDs per sequence
    const int per = a.tiles / (2 * X);            // long (and short) tiles per XCD run
    const int xcd = bid & 7, jj = bid >> 3;
    group = xcd / X;
    tile = jj < per ? per * (xcd % X) + jj : (a.tiles >> 1) + per * (xcd % X) + (jj - per);
  }
  if (tile >= a.tiles) return;
  const int q = group * g + j;

  // the query's visible length and sequence base: scalar loads waited for
  // together (one round trip before the first key load)
  const int n = a.n_visible[q];
  const int64_t sbase = a.seq_base[q];
  asm volatile("" ::"s"(n), "s"(sbase));
  const int c = max(0, n - a.swa);
  // with two workgroups per CU, the one dispatched first (the first half of
  // the tile indices) streams faster, so it gets the longer tile
  const int half_t = a.tiles >> 1;
  const int t_long = a.tile_pos + a.tile_extra, t_short = a.tile_pos - a.tile_extra;
  const int p_begin = tile < half_t ? tile * t_long : half_t * t_long + (tile - half_t) * t_short;
  if (p_begin >= c) return;
  const int p_end = min(p_begin + (tile < half_t ? t_long : t_short), c);
  const int nsteps = (p_end - p_begin + 15) >> 4;

  v8h qf[HT][KC];
  float wv[HT][4];
  const uint8_t* qp = a.idx_q + (int64_t)q * a.hi * RB;

  // buffer descriptor over this sequence's candidate keys, built from
  // wave-uniform scalars (rows >= c read as zero)
  // (paged: over the whole plane; rows >= c are then masked per lane)
  const int64_t kbase = PG ? 0 : sbase;
  const uint32_t krows = PG ? (uint32_t)a.rows : (uint32_t)c;
  const uint64_t kaddr = (uint64_t)(uintptr_t)(a.idx_k + kbase * RB);
  const v4u rsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)kaddr),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(kaddr >> 32)) & 0xFFFFu,
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(krows * RB)), 0x00020000u};
  v4u srsrc = rsrc;                     // FP4: the candidates' scale rows
  if constexpr (F4) {
    const uint64_t saddr = (uint64_t)(uintptr_t)(a.idx_k_scales + kbase * SB);
    srsrc = v4u{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)saddr),
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(saddr >> 32)) & 0xFFFFu,
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(krows * SB)), 0x00020000u};
  }
  const int pg0 = PG ? p_begin >> a.page_shift : 0;   // the tile's first page
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Whole-line key loads.  The reduction dimension is split into 16-byte
  // chunks: MFMA lane (col, gq) needs chunk gq (and, for d = 128, chunk 4 + gq)
  // of row col.  A load instruction instead gives lane l one chunk of a row so
  // that it covers whole 128-byte lines, and the chunk index is rotated by the
  // row so that the MFMA-side LDS reads of 8 consecutive lanes (8 rows, one
  // chunk) fall on 8 different 16-byte bank groups.
  //   d = 128: instruction h holds rows 8h .. 8h+7; lane l = 8a + j holds row
  //            8h + a, chunk (j - a) mod 8.
  //   d = 64:  one instruction holds the 16 rows; lane l = 4r + j holds row r,
  //            chunk (j - (r >> 1)) mod 4.
  const int ld_row = D == 128 ? lane >> 3 : lane >> 2;
  const int ld_chunk = D == 128 ? ((lane & 7) - (lane >> 3)) & 7 : ((lane & 3) - ((lane >> 3) & 3)) & 3;
  int rd_pos[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int ch = gq + 4 * h;               // the chunk this lane's MFMA operand needs
    rd_pos[h] = D == 128 ? (col >> 3) * 64 + (col & 7) * 8 + ((ch + (col & 7)) & 7)
                         : col * 4 + ((ch + ((col >> 1) & 3)) & 3);
  }

  // this wave's steps are s_k = wave + NW k, k < ns, streamed through R LDS
  // slots with R - 1 steps of direct-to-LDS loads in flight.  The loads are
  // issued as inline asm so that the compiler neither tracks them (it would
  // wait for every one of them before each LDS read) nor moves them; the
  // waits below count them explicitly (vector-memory ops retire in order).
  // (wave-uniform: the loop below branches on scalars, with no exec masking)
  const int ns = __builtin_amdgcn_readfirstlane(wave_u < nsteps ? (nsteps - wave_u + NW - 1) / NW : 0);
  // step k goes to ring slot sl = k mod R; every call site passes sl as a
  // constant (the loop is unrolled by R), so slot addresses are immediates
  auto issue = [&](int k, int sl) {
    const int row0 = p_begin + (wave + NW * k) * 16;
    // the step's 16 rows are 16-aligned, so they share one page
    uint32_t prow0 = (uint32_t)row0;
    if constexpr (PG)
      prow0 = ((uint32_t)s_pg[(row0 >> a.page_shift) - pg0] << a.page_shift) |
              ((uint32_t)row0 & ((1u << a.page_shift) - 1u));
    const uint32_t slot = (uint32_t)(uintptr_t)(lds_void*)&s_ring[wave_u][sl][0];
    if constexpr (F4) {
      // 16 rows of 64 code bytes: one whole KiB (lane l: row l & 15, bytes 16 (l >> 4) .. +16)
      const uint32_t row = !PG || row0 + col < c ? (prow0 + col) * RB : kOob;
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                   :: "s"(m0), "v"(row + gq * 16), "s"(rsrc) : "memory", "m0");
      // the step's 16 x 8 scale bytes: dword `lane` of them for lanes < 32
      const uint32_t m1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(slot + 1024));
      const uint32_t so = lane < 32 && (!PG || row0 + (lane >> 1) < c) ? prow0 * SB + lane * 4 : kOob;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen nt lds"
                   :: "s"(m1), "v"(so), "s"(srsrc) : "memory", "m0");
    } else {
      // each load instruction reads whole 128-byte lines (1 KiB contiguous):
      // lane l -> (row ld_row + 8h or 16 rows of 64 B, chunk ld_chunk), stored
      // at LDS position l of the instruction's KiB
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int r = ld_row + 8 * h;
        const uint32_t row = !PG || row0 + r < c ? (prow0 + r) * RB + ld_chunk * 16 : kOob;
        const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(slot + h * 1024));
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :: "s"(m0), "v"(row), "s"(rsrc) : "memory", "m0");
      }
    }
  };
  // fetch: wait until step k has landed (keeping the younger steps in
  // flight), refill the ring, read the lane's bytes and convert to f16
  auto fetch = [&](int k, int sl, v8h* kf) {
    if (k + R - 1 < ns) {
      wait_lgkmcnt0();                 // the slot's previous reads are done
      issue(k + R - 1, (sl + R - 1) % R);
      wait_vmcnt<(R - 1) * LPS>();     // step k has landed; R - 1 younger in flight
    } else {
      wait_vmcnt<0>();
    }
    const uint8_t* slot = &s_ring[wave_u][sl][0];
    if constexpr (F4) {
      // the lane's 32 channels: four code dwords (8 channels each) and the
      // scales of its two 16-channel groups (row col, scale bytes 2gq, 2gq + 1)
      const v4u x = *reinterpret_cast<const v4u*>(slot + lane * 16);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(slot + 1024 + (col * 2 + (gq >> 1)) * 4);
      const v2h sc = fp4_pair_scales(sw, gq & 1);
      const v2h s0 = {sc[0], sc[0]}, s1 = {sc[1], sc[1]};
      kf[0] = fp4x8_to_v8h(x[0], s0);
      kf[1] = fp4x8_to_v8h(x[1], s0);
      kf[2] = fp4x8_to_v8h(x[2], s1);
      kf[3] = fp4x8_to_v8h(x[3], s1);
    } else {
      // the lane's raw E4M3 bytes (d = 64: 16 of them, the rest zero) in
      // kf[0], kf[1]; the other fragments are unused
#pragma unroll
      for (int h = 0; h < NH; ++h)
        kf[h] = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(slot + rd_pos[h] * 16));
      if constexpr (NH == 1) kf[1] = __builtin_bit_cast(v8h, (v4u{0u, 0u, 0u, 0u}));
    }
  };
  auto contract = [&](const v8h* kf, v4f* acc) {
#pragma unroll
    for (int t = 0; t < HT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (F4) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
        for (int t = 0; t < HT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[t][kc], kf[kc], acc[t], 0, 0, 0);
      }
    } else {
      const v8i kb = cat_v8i(__builtin_bit_cast(v4u, kf[0]), __builtin_bit_cast(v4u, kf[1]));
#pragma unroll
      for (int t = 0; t < HT; ++t)
        acc[t] = mfma_fp8_k128(cat_v8i(__builtin_bit_cast(v4u, qf[t][0]), __builtin_bit_cast(v4u, qf[t][1])), kb, acc[t]);
    }
  };
  // last: the wave's final step, the only one that can reach past c (the
  // tile's last step is the last step of the wave that has it)
  auto epilogue = [&](const v4f* acc, int k, bool last) {
    // four independent partial sums (no 16-long dependent chain)
    float pp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < HT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[i] += wv[t][i] * fmaxf(acc[t][i], 0.0f);
    }
    const float part = sum_rows4((pp[0] + pp[1]) + (pp[2] + pp[3]));
    const int s = wave + NW * k;
    const int p0 = p_begin + s * 16;
    // positions >= c (only in a wave's last step) score -inf
    float v = part;
    if (last) v = p0 + col < c ? part : -__builtin_inff();
    // every lane group holds the same 16 sums: group 0 writes the position
    // keys (key 0, which no score has, for positions >= c) straight to the
    // row (64 bytes per step; staging them in LDS cost a third workgroup per
    // CU, which the compute-bound many-token scans need)
    if constexpr (PS)
      if (gq == 0) a.pkey[(int64_t)q * a.ld_pkey + p0 + col] = !last || p0 + col < c ? order_key(part) : 0u;
    v = max_lanes8(v);
    if (lane < 16 && (lane & 7) == 0) s_bs[s * 2 + (lane >> 3)] = v;
  };

  // software pipeline: the MFMAs of step k run while the VALU finishes
  // step k - 1 (epilogue) and prepares step k + 1 (LDS read; FP4: the
  // conversion to f16), none of which depends on the MFMAs in flight
  // The query (H_i x d fp8, one contiguous block) and the head weights come
  // in by direct-to-LDS loads issued before the first key loads, so they land
  // first: the explicit wait below covers them while the keys stay in flight
  // (a compiler-tracked vector load here would make the compiler wait for
  // every load before it, key loads included, and stall the whole stream).
  {
    const uint64_t qaddr = (uint64_t)(uintptr_t)qp;
    const v4u qrsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qaddr),
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(qaddr >> 32)) & 0xFFFFu,
                       (uint32_t)__builtin_amdgcn_readfirstlane(a.hi * RB), 0x00020000u};
    const int qvec = (a.hi * RB + 1023) >> 10;         // 1 KiB per load instruction
    for (int v = wave_u; v < qvec; v += NW) {
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(uintptr_t)(lds_void*)s_q + v * 1024));
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0), "v"((uint32_t)(v * 1024 + lane * 16)), "s"(qrsrc) : "memory", "m0");
    }
    if constexpr (F4) {
      // the query's scale rows (H_i x 8 bytes) after its codes, 256 bytes per load
      const uint64_t saddr = (uint64_t)(uintptr_t)(a.idx_q_scales + (int64_t)q * a.hi * SB);
      const v4u qsrsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)saddr),
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(saddr >> 32)) & 0xFFFFu,
                          (uint32_t)__builtin_amdgcn_readfirstlane(a.hi * SB), 0x00020000u};
      const int svec = (a.hi * SB + 255) >> 8;
      for (int v = wave_u; v < svec; v += NW) {
        const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((uint32_t)(uintptr_t)(lds_void*)s_q + 64 * RB + v * 256));
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :: "s"(m0), "v"((uint32_t)(v * 256 + lane * 4)), "s"(qsrsrc) : "memory", "m0");
      }
    }
    if (wave_u == 0) {
      // the head weights, 4 bytes per lane (weights past H_i read as zero)
      const uint64_t waddr = (uint64_t)(uintptr_t)(a.idx_w + (int64_t)q * a.hi);
      const v4u wrsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)waddr),
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(waddr >> 32)) & 0xFFFFu,
                         (uint32_t)__builtin_amdgcn_readfirstlane(a.hi * 4), 0x00020000u};
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)s_w);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                   :: "s"(m0), "v"((uint32_t)(lane * 4)), "s"(wrsrc) : "memory", "m0");
    }
  }
  if constexpr (PG) {
    // the tile's page ids into LDS before the first key load
    const int npg = ((p_end - 1) >> a.page_shift) - pg0 + 1;
    for (int t = tid; t < npg; t += NT) s_pg[t] = a.pages[sbase + pg0 + t];
    __syncthreads();
  }
  const int pro = min(R - 1, ns);
#pragma unroll
  for (int k = 0; k < R - 1; ++k)
    if (k < pro) issue(k, k);
  if (pro == R - 1) wait_vmcnt<(R - 1) * LPS>();   // the query loads (older) have landed
  else wait_vmcnt<0>();
  __syncthreads();

  // query fragments (f16) and head weights for this lane, from LDS
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int h = t * 16 + col;
    const bool live = h < a.hi;
    v4u qx = {0u, 0u, 0u, 0u};
    v2h qsc = {(_Float16)0.0f, (_Float16)0.0f};
    if constexpr (F4) {
      // head h's channels 32gq .. +32 (the keys' k-slot map) and their scales
      const int hc = min(h, a.hi - 1);
      qx = *reinterpret_cast<const v4u*>(&s_q[hc * RB + gq * 16]);
      qsc = fp4_pair_scales(*reinterpret_cast<const uint32_t*>(&s_q[64 * RB + hc * SB + (gq >> 1) * 4]), gq & 1);
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (F4) {
        const _Float16 s = kc < 2 ? qsc[0] : qsc[1];
        qf[t][kc] = fp4x8_to_v8h(live ? qx[kc] : 0u, v2h{s, s});
      } else {
        // raw E4M3 bytes, the keys' byte -> k-slot map: chunk gq (and, for
        // d = 128, chunk 4 + gq) of 16 bytes in qf[t][0], qf[t][1]
        v4u x = {0u, 0u, 0u, 0u};
        if (kc < NH && live) x = *reinterpret_cast<const v4u*>(&s_q[h * D + key_chunk<D>(gq, kc)]);
        qf[t][kc] = __builtin_bit_cast(v8h, x);
      }
      // keep the converted fragments resident: without this the compiler
      // re-converts them inside the loop to save registers
      if (F4 || kc < 2) asm volatile("" : "+v"(qf[t][kc]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = s_w[t * 16 + gq * 4 + i];
  }
  if (ns > 0) {
    // ping-pong between two fragment / accumulator sets (no register copies
    // of MFMA results, which would stall on the MFMAs in flight)
    v8h kfa[KC], kfb[KC];
    v4f acca[HT], accb[HT];
    fetch(0, 0, kfa);
    for (int k0 = 0;; k0 += R) {
#pragma unroll
      for (int u = 0; u < R; u += 2) {
        const int k = k0 + u;                    // step k uses slot u, step k + 1 slot u + 1
        contract(kfa, acca);                     // step k
        if (k > 0) epilogue(accb, k - 1, false);
        if (k + 1 >= ns) { epilogue(acca, k, true); goto stream_done; }
        fetch(k + 1, u + 1, kfb);
        contract(kfb, accb);                     // step k + 1
        epilogue(acca, k, false);
        if (k + 2 >= ns) { epilogue(accb, k + 1, true); goto stream_done; }
        fetch(k + 2, (u + 2) % R, kfa);
      }
    }
  stream_done:;
  }
  __syncthreads();
  // block scores of the tile, one coalesced store
  float* bs = a.bscore + (int64_t)q * a.ld + (p_begin >> 3);
  const int nblk = (p_end - p_begin + 7) >> 3;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  if (a.gkey) {
    // and the group keys: 16 lanes hold one group's blocks (the tile starts
    // at a group boundary; a partial last group reads 0 past the tile)
    uint32_t* gk = a.gkey + (int64_t)q * a.ld_gkey + (p_begin >> 7);
    const int nblk16 = (nblk + kGroupBlocks - 1) & ~(kGroupBlocks - 1);
    for (int i = tid; i < nblk16; i += NT) {
      const bool live = i < nblk;
      const float v = s_bs[min(i, nblk - 1)];
      const uint32_t k = live ? order_key(v) : 0u;
      if (live) {
        bs[i] = v;
        lo = min(lo, k);
        hi = max(hi, k);
      }
      uint32_t m = k;
#pragma unroll
      for (int d = 1; d < kGroupBlocks; d <<= 1) m = max(m, (uint32_t)__shfl_xor(m, d, 64));
      if ((i & (kGroupBlocks - 1)) == 0) gk[i >> 4] = m;
    }
  } else {
    for (int i = tid; i < nblk; i += NT) {
      const float v = s_bs[i];
      bs[i] = v;
      lo = min(lo, order_key(v));
      hi = max(hi, order_key(v));
    }
  }
  if (a.pool_ws) {
    // the tile's key range for the pool select, and (tile 0) its histogram cleared
    uint32_t* pw = a.pool_ws + (int64_t)q * a.pool_ws_stride;
    if (tile == 0) {
      for (int i = tid * 4; i < kHistBins; i += NT * 4) *reinterpret_cast<v4u*>(pw + i) = v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      lo = min(lo, (uint32_t)__shfl_xor(lo, d, 64));
      hi = max(hi, (uint32_t)__shfl_xor(hi, d, 64));
    }
    __shared__ uint32_t s_mm[2 * NW];
    if (lane == 0) { s_mm[wave] = lo; s_mm[NW + wave] = hi; }
    __syncthreads();
    if (tid == 0) {
      uint32_t l2 = s_mm[0], h2 = s_mm[NW];
#pragma unroll
      for (int i = 1; i < NW; ++i) { l2 = min(l2, s_mm[i]); h2 = max(h2, s_mm[NW + i]); }
      *reinterpret_cast<v2u*>(pw + kHistBins + 2 * tile) = v2u{l2, h2};
    }
  }
}

template <int D, int R, int NW, bool F4, bool PG = false, bool PS = false>
hipError_t launch_drw(const ScanArgs& a, hipStream_t s) {
  const int ht = (a.hi + 15) / 16;
  const int units = ((a.n_q / a.g) * a.tiles + 7) / 8 * 8;
  const dim3 grid((unsigned)(units * a.g)), block(64 * NW);
  switch (ht) {
    case 1: hipLaunchKernelGGL((k_scan<D, 1, R, NW, F4, PG, PS>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_scan<D, 2, R, NW, F4, PG, PS>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_scan<D, 3, R, NW, F4, PG, PS>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_scan<D, 4, R, NW, F4, PG, PS>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int D, bool F4>
hipError_t launch_d(const ScanArgs& a, hipStream_t s) {
  // position keys, paged keys: the default ring and wave count only
  if (a.pkey)
    return a.pages ? launch_drw<D, kScanPrefetch, kScanWaves, F4, true, true>(a, s)
                   : launch_drw<D, kScanPrefetch, kScanWaves, F4, false, true>(a, s);
  if (a.pages) return launch_drw<D, kScanPrefetch, kScanWaves, F4, true>(a, s);
  // LDS ring slots per wave (steps in flight + 1) and waves per workgroup
  if (a.waves == 8) {
    if (a.prefetch == 8) return launch_drw<D, 8, 8, F4>(a, s);
    return a.prefetch == 6 ? launch_drw<D, 6, 8, F4>(a, s) : launch_drw<D, 4, 8, F4>(a, s);
  }
  if (a.prefetch == 8) return launch_drw<D, 8, 4, F4>(a, s);
  return a.prefetch == 6 ? launch_drw<D, 6, 4, F4>(a, s) : launch_drw<D, 4, 4, F4>(a, s);
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.tiles == 0) return hipSuccess;
  if (a.pkey && (a.ld_pkey % 32 || ((uintptr_t)a.pkey & 15))) return hipErrorInvalidValue;
  if (a.tile_pos > kMaxTilePos || a.tile_pos % 64) return hipErrorInvalidValue;
  if (a.pages && (a.tile_extra % 16 || a.page_shift < 4 || a.page_shift > 16 || a.rows * (a.d / (a.idx_k_scales ? 2 : 1)) > 0xFFFFFF00LL))
    return hipErrorInvalidValue;
  if (a.tile_extra < 0 || a.tile_extra % 8 || a.tile_extra >= a.tile_pos ||
      a.tile_pos + a.tile_extra > kMaxTilePos || (a.tile_extra && (a.tiles & 1)))
    return hipErrorInvalidValue;
  if (a.gkey && (a.tile_pos % (8 * kGroupBlocks) || a.tile_extra % (8 * kGroupBlocks) || a.ld_gkey < 4))
    return hipErrorInvalidValue;
  if (a.idx_k_scales) {
    if (a.d != 128 || !a.idx_q_scales) return hipErrorInvalidValue;
    return launch_d<128, true>(a, s);
  }
  return a.d == 64 ? launch_d<64, false>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace csa2
