// Core attention over the kept FP4 entries and the bf16 sliding window, with
// one softmax and a 512-wide latent output per head (MLA-absorbed).
//
// Follows "DeepSeek-V4.1-Flash 梗概" §3.2 (heterogeneous KV: the same main Q
// attends the sparse main-KV branch and the uncompressed window branch and
// the two are merged; mode table: Reuse layers change only Q) and §4 of the
// newsaint.id page (FP4 main KV dequantised just before attention).  The key
// of a sparse entry is [dequantised latent (512) || bf16 rope (64)] and its
// value is the dequantised latent; a window row supplies both from bf16.
// The FP4 scales cover 16 channels, or 32 in the group-32 codec variant (the
// akhunji.com page, "Microscopic FP4 (E2M1) Cache Compression"): a gathered
// 16-channel item then reads the scale byte of its 32-channel group.
//
// Mapping (gfx950): a workgroup = 4 waves = one query x up to 64 heads (one
// wave per 16 heads; waves past the last head only help gather) x one split
// of the entry list.  Entries stream in tiles of 32:
//  * the split's cache rows are resolved into LDS once; each tile's raw
//    bytes (FP4 codes + E4M3 scale, or bf16 window values, and the rope) are
//    loaded into registers one tile ahead, so the gather of tile t+1 is in
//    flight while tile t is contracted;
//  * the raw tile is dequantised into one row-major f16 image in LDS (FP4 x
//    E4M3 values are exact in f16; bf16 window / rope / query values are exact
//    in f16 inside its normal range, the reason for the |x| < 65504 bound);
//  * Q.K^T: v_mfma_f32_16x16x32_f16 with the tile as A (rows = entries) and
//    the wave's 16 query heads as B (held in registers), giving S^T whose lane
//    layout is exactly the A layout P.V needs, so P never leaves registers;
//  * online softmax in the exp2 domain, P rounded to f16 (bf16 would cost
//    about 2^-9 relative per weight); P.V with v_mfma_f32_16x16x32_f16 whose
//    value operand is read from the same row-major image with the gfx950 LDS
//    transpose read (ds_read_b64_tr_b16), into 32 accumulator tiles
//    (16 heads x 512 dims);
//  * with several splits per query, unnormalised partials (o, m, l) are
//    merged by k_attend_combine with a log-sum-exp rescale.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kTile = kAttendTile;        // 32 entries
constexpr int kNW = kAttendWaves;         // waves per workgroup, 16 heads each
constexpr int kNT = 64 * kNW;
constexpr int kKS = kKeyDim + 8;          // f16 row stride of the tile image
constexpr int kMaxSplit = 2048 + 1024;    // entries of one split (topk + swa bounds)
constexpr int kRowPer = (kMaxSplit + kNT - 1) / kNT;   // kept positions per thread

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// bf16 pair -> f16 pair.  Exact for values inside the f16 range (the ABI's
// |x| < 65504 precondition); round-toward-zero only matters outside it.
__device__ __forceinline__ uint32_t bf16x2_to_h2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)));
}

// Four code bytes (eight E2M1 values, low nibble first) times an E4M3 scale,
// as four f16 pairs.  The gfx950 conversion at scale 1.0 is exact, and so is
// the f16 product: E2M1 x E4M3 needs at most 6 significant bits and lies in
// [2^-13, 2688].
template <int B>
__device__ __forceinline__ uint32_t fp4_byte_h2(uint32_t word, v2h s2) {
  const v2h x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, B);
  return __builtin_bit_cast(uint32_t, x * s2);
}

constexpr int kItems = kTile * 32 / kNT;      // (entry, 16-channel group) items per thread
constexpr int kRopeItems = kTile * 8 / kNT;   // (entry, 8-channel rope chunk) items per thread

// One tile's raw bytes held by a thread, loaded a tile ahead: an item keeps
// its 8 code bytes in c.xy and the aligned word holding its scale byte in
// c.z; a rope chunk comes from the cache (r) or a window row (rw), the other
// reading zeros.  Window items' latent values (at most W rows per query,
// bf16) are read when the tile is stored.
struct RawTile {
  v4u c[kItems];
  v4u r[kRopeItems];
  v4u rw[kRopeItems];
};

// The query's sources as buffer resources over exactly its rows, so that a
// load at offset kOob returns zeros: every load below is issued for every
// item, masked by its offset instead of a branch (a load inside a divergent
// branch waits for itself, and for everything issued before it), and no
// loaded value is touched before the tile is stored.
constexpr uint32_t kOob = 0xFFFFFF00u;
struct TileSrc {
  __amdgpu_buffer_rsrc_t codes, scales, rope, win;
  uint32_t sbytes;           // scale bytes per entry (32, or 16 with 32-channel groups)
  int gshift;                // 16-channel item -> its scale byte: item >> gshift
};

__device__ __forceinline__ TileSrc tile_src(const AttendArgs& a, int64_t seq_base, int64_t swa_base, int n, int w) {
  TileSrc s;
  s.codes = make_rsrc(a.kv_codes + seq_base * kCodeBytes, (uint32_t)n * kCodeBytes);
  s.gshift = a.kv_gshift;
  s.sbytes = (uint32_t)kScaleBytes >> a.kv_gshift;
  s.scales = make_rsrc(a.kv_scales + seq_base * s.sbytes, (uint32_t)n * s.sbytes);
  s.rope = make_rsrc(a.kv_rope + seq_base * kRope, (uint32_t)n * kRope * 2);
  s.win = make_rsrc(a.swa_kv + swa_base * kKeyDim, (uint32_t)w * kKeyDim * 2);
  return s;
}

// The row ids of a thread's items in a tile of ne entries: rows[e] >= 0
// is a sparse entry at position rows[e] (cache row seq_base + pos), rows[e]
// < 0 the window row swa_base + (-1 - rows[e]); entries e >= ne read as
// kNoRow.  All LDS reads first, then the selects.
constexpr int32_t kNoRow = 0x7FFFFFFF;
struct TileRows {
  int32_t it[kItems];
  int32_t rp[kRopeItems];
};

__device__ __forceinline__ TileRows tile_rows(const int32_t* rows, int ne, int tid) {
  TileRows t;
#pragma unroll
  for (int k = 0; k < kItems; ++k) t.it[k] = rows[max(0, min((tid + k * kNT) >> 5, ne - 1))];
#pragma unroll
  for (int k = 0; k < kRopeItems; ++k) t.rp[k] = rows[max(0, min((tid + k * kNT) >> 3, ne - 1))];
#pragma unroll
  for (int k = 0; k < kItems; ++k) asm volatile("" : "+v"(t.it[k]));
#pragma unroll
  for (int k = 0; k < kRopeItems; ++k) asm volatile("" : "+v"(t.rp[k]));
#pragma unroll
  for (int k = 0; k < kItems; ++k) t.it[k] = ((tid + k * kNT) >> 5) < ne ? t.it[k] : kNoRow;
#pragma unroll
  for (int k = 0; k < kRopeItems; ++k) t.rp[k] = ((tid + k * kNT) >> 3) < ne ? t.rp[k] : kNoRow;
  return t;
}

__device__ __forceinline__ void load_tile(const TileSrc& src, const int32_t* rows, int ne, int tid, RawTile& t) {
  const TileRows tr = tile_rows(rows, ne, tid);
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int grp = (tid + k * kNT) & 31;
    const int32_t r = tr.it[k];
    const bool sp = r >= 0 && r != kNoRow;
    const v2u cw = __builtin_amdgcn_raw_buffer_load_b64(src.codes, sp ? (uint32_t)r * kCodeBytes + grp * 8 : kOob, 0, 0);
    const uint32_t sw = __builtin_amdgcn_raw_buffer_load_b32(
        src.scales, sp ? ((uint32_t)r * src.sbytes + (grp >> src.gshift)) & ~3u : kOob, 0, 0);
    t.c[k] = v4u{cw[0], cw[1], sw, 0u};
  }
#pragma unroll
  for (int k = 0; k < kRopeItems; ++k) {
    const int ch = (tid + k * kNT) & 7;
    const int32_t r = tr.rp[k];
    const uint32_t osp = r >= 0 && r != kNoRow ? (uint32_t)r * (kRope * 2) + ch * 16 : kOob;
    const uint32_t ow = r < 0 ? (uint32_t)(-1 - r) * (kKeyDim * 2) + kLatent * 2 + ch * 16 : kOob;
    t.r[k] = buf_load16(src.rope, osp);
    t.rw[k] = buf_load16(src.win, ow);
  }
}

// Dequantise a tile into the f16 image (rows past the tile's end are 0).  The
// window rows' bf16 values are loaded here, all items at once.
__device__ __forceinline__ void store_tile(const TileSrc& src, const int32_t* rows, int ne, bool has_win,
                                           const RawTile& t, int tid, _Float16* s_k) {
  const TileRows tr = tile_rows(rows, ne, tid);
  v4u w0[kItems], w1[kItems];
  if (has_win) {
    // a tile that reaches into the window (uniform): every item's window
    // load is issued before the first is used
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int grp = (tid + k * kNT) & 31;
      const uint32_t ow = tr.it[k] < 0 ? (uint32_t)(-1 - tr.it[k]) * (kKeyDim * 2) + grp * 32 : kOob;
      w0[k] = buf_load16(src.win, ow);
      w1[k] = buf_load16(src.win, ow + 16);
    }
#pragma unroll
    for (int k = 0; k < kItems; ++k) asm volatile("" : "+v"(w0[k]), "+v"(w1[k]));
  } else {
#pragma unroll
    for (int k = 0; k < kItems; ++k) { w0[k] = v4u{0u, 0u, 0u, 0u}; w1[k] = w0[k]; }
  }
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int it = tid + k * kNT, e = it >> 5, grp = it & 31;
    v4u h0, h1;
    if (tr.it[k] < 0) {
      h0 = v4u{bf16x2_to_h2(w0[k][0]), bf16x2_to_h2(w0[k][1]), bf16x2_to_h2(w0[k][2]), bf16x2_to_h2(w0[k][3])};
      h1 = v4u{bf16x2_to_h2(w1[k][0]), bf16x2_to_h2(w1[k][1]), bf16x2_to_h2(w1[k][2]), bf16x2_to_h2(w1[k][3])};
    } else {
      const _Float16 sh = (_Float16)e4m3_to_float((t.c[k][2] >> (8 * ((grp >> src.gshift) & 3))) & 0xFFu);  // exact
      const v2h s2 = {sh, sh};
      const uint32_t c0 = t.c[k][0], c1 = t.c[k][1];
      h0 = v4u{fp4_byte_h2<0>(c0, s2), fp4_byte_h2<1>(c0, s2), fp4_byte_h2<2>(c0, s2), fp4_byte_h2<3>(c0, s2)};
      h1 = v4u{fp4_byte_h2<0>(c1, s2), fp4_byte_h2<1>(c1, s2), fp4_byte_h2<2>(c1, s2), fp4_byte_h2<3>(c1, s2)};
    }
    v4u* dk = reinterpret_cast<v4u*>(s_k + e * kKS + grp * 16);
    dk[0] = h0;
    dk[1] = h1;
  }
#pragma unroll
  for (int k = 0; k < kRopeItems; ++k) {
    const int it = tid + k * kNT, e = it >> 3, ch = it & 7;
    const v4u r = t.r[k] | t.rw[k];
    *reinterpret_cast<v4u*>(s_k + e * kKS + kLatent + ch * 8) =
        v4u{bf16x2_to_h2(r[0]), bf16x2_to_h2(r[1]), bf16x2_to_h2(r[2]), bf16x2_to_h2(r[3])};
  }
}

__global__ __launch_bounds__(kNT) void k_attend(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 s_k[kTile * kKS];
  __shared__ __attribute__((aligned(16))) _Float16 s_q[kNW * 16 * kKS];   // per wave: 16 heads x 576
  __shared__ int32_t s_row[kMaxSplit];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, col = lane & 15;
  const int S = a.splits, HG = a.head_groups;
  const int q = blockIdx.x / (HG * S);
  const int hg = (blockIdx.x / S) % HG;
  const int sp = blockIdx.x % S;
  const int H = a.heads;
  const int head0 = (hg * kNW + wave) * 16;
  const bool active = head0 < H;           // wave-uniform

  const int e_begin = sp * a.split_entries;
  const int32_t* tk = a.topk_pos + (int64_t)q * a.topk;
  int32_t tkv[kRowPer];
  {
    const int e_lim = min(a.topk, e_begin + a.split_entries);
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const int e = e_begin + tid + j * kNT;
      const int32_t v = tk[min(e, a.topk - 1)];      // the row always holds topk entries
      tkv[j] = e < e_lim ? v : 0;
    }
  }
  // the wave's 16 query heads as f16 rows [head][576] (the B operand of
  // Q.K^T): all 18 loads per lane issued before the first use
  constexpr int kQv = 16 * (kKeyDim / 8) / 64;
  v4u rq[kQv];
  if (active) {
#pragma unroll
    for (int j = 0; j < kQv; ++j) {
      const int i = lane + 64 * j, hh = i / (kKeyDim / 8), d = (i % (kKeyDim / 8)) * 8;
      // heads past H (H a multiple of 8, not 16) read as zero rows
      const int64_t qh = (int64_t)q * H + min(head0 + hh, H - 1);
      const uint16_t* src = d < kLatent ? a.q_lat + qh * kLatent + d : a.q_rope + qh * kRope + (d - kLatent);
      rq[j] = *reinterpret_cast<const v4u*>(src);
      if (head0 + hh >= H) rq[j] = v4u{0u, 0u, 0u, 0u};
    }
  }
  const int n = load_uniform(a.n_visible + q);
  const int c = max(0, n - a.swa);
  const int Es = min(load_uniform(a.topk_count + q), a.topk);
  const int E = Es + (n - c);
  const int e_end = min(E, e_begin + a.split_entries);
  const int64_t sbase = load_uniform(a.seq_base + q);
  // paged main KV: the kept positions become rows of the whole planes (one
  // page id per position, loaded unconditionally from a clamped slot)
  const bool paged = a.pages != nullptr;
  if (paged && c > 0) {
    int32_t pg[kRowPer];
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) pg[j] = a.pages[sbase + (min(max(tkv[j], 0), c - 1) >> a.page_shift)];
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) asm volatile("" : "+v"(pg[j]));
#pragma unroll
    for (int j = 0; j < kRowPer; ++j)
      tkv[j] = (int32_t)(((uint32_t)pg[j] << a.page_shift) | ((uint32_t)tkv[j] & ((1u << a.page_shift) - 1u)));
  }
  const TileSrc src = tile_src(a, paged ? 0 : sbase, load_uniform(a.swa_base + q), paged ? (int)a.rows : n, n - c);

  {
    // the split's kept positions: the row always holds `topk` entries, so
    // these loads were issued before the counts (a.n_visible, a.topk_count)
    // they are filtered by arrived
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const int e = e_begin + tid + j * kNT;
      if (e < e_end) s_row[e - e_begin] = e < Es ? tkv[j] : -1 - (e - Es);
    }
  }
  __syncthreads();
  // raw tiles two deep: tiles t and t+1 are in flight while t-1 is contracted
  RawTile ra, rb;
  // (unconditional: a tile past the split's end loads zeros)
  load_tile(src, s_row, min(kTile, e_end - e_begin), tid, ra);
  load_tile(src, s_row + kTile, min(kTile, e_end - e_begin - kTile), tid, rb);
  // the query into LDS while the first tiles are in flight (read after the
  // first tile's barriers)
  if (active) {
    _Float16* sq = s_q + wave * 16 * kKS;
#pragma unroll
    for (int j = 0; j < kQv; ++j) {
      const int i = lane + 64 * j, hh = i / (kKeyDim / 8), d = (i % (kKeyDim / 8)) * 8;
      *reinterpret_cast<v4u*>(sq + hh * kKS + d) =
          v4u{bf16x2_to_h2(rq[j][0]), bf16x2_to_h2(rq[j][1]), bf16x2_to_h2(rq[j][2]), bf16x2_to_h2(rq[j][3])};
    }
  }
  const _Float16* sqw = s_q + (wave * 16 + col) * kKS + gq * 8;

  float m = -__builtin_inff(), l = 0.0f;
  v4f o[kLatent / 16];
#pragma unroll
  for (int nt = 0; nt < kLatent / 16; ++nt) o[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto tile = [&](RawTile& raw, int e0) {
    const int ne = min(kTile, e_end - e0);
    __syncthreads();                         // the previous tile's reads of s_k are done
    store_tile(src, s_row + (e0 - e_begin), ne, e0 + ne > Es, raw, tid, s_k);
    const int e2 = e0 + 2 * kTile;           // this register set's next tile
    if (e2 < e_end) load_tile(src, s_row + (e2 - e_begin), min(kTile, e_end - e2), tid, raw);
    __syncthreads();
    if (!active) return;

    // ---- S^T = K_tile . Q^T  (rows: entries, cols: heads)
    v4f s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kKeyDim / 32; ++ks) {
      const v8h k0 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(s_k + col * kKS + ks * 32 + gq * 8));
      const v8h k1 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(s_k + (16 + col) * kKS + ks * 32 + gq * 8));
      const v8h qb = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(sqw + ks * 32));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qb, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qb, s1, 0, 0, 0);
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
    // ---- O += P . V   (k-slots: entries 4gq..4gq+3, then 16+4gq..16+4gq+3;
    //      the transpose read hands lane `col` four entries of dim 16nt+col)
    const int ra = 4 * gq + (col >> 2), cb = 4 * (col & 3);
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s_k + ra * kKS + nt * 16 + cb));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s_k + (16 + ra) * kKS + nt * 16 + cb));
      const v8h vb = __builtin_bit_cast(v8h, (v4u{__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1],
                                                  __builtin_bit_cast(v2u, hi)[0], __builtin_bit_cast(v2u, hi)[1]}));
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vb, o[nt], 0, 0, 0);
    }
  };
  for (int e0 = e_begin; e0 < e_end; e0 += 2 * kTile) {
    tile(ra, e0);
    if (e0 + kTile < e_end) tile(rb, e0 + kTile);
  }

  if (!active) return;

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
        if (head0 + 4 * gq + i < H)
          a.out[((int64_t)q * H + head0 + 4 * gq + i) * kLatent + nt * 16 + col] = o[nt][i] * inv[i];
    }
    if (a.lse && gq == 0 && head0 + col < H)
      a.lse[(int64_t)q * H + head0 + col] = l > 0.0f ? (m + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
  } else {
    // partial o of the wave's 16 heads in the accumulators' own layout
    // [nt][lane][4] (one 1 KiB coalesced store per nt); k_attend_combine
    // reads it back in the same layout
    // (partials cover the heads padded to a multiple of 16)
    const int HB = (H + 15) / 16;
    float* po = a.part_o + (((int64_t)q * S + sp) * HB + head0 / 16) * (kLatent * 16);
#pragma unroll
    for (int nt = 0; nt < kLatent / 16; ++nt)
      *reinterpret_cast<v4f*>(po + (nt * 64 + lane) * 4) = o[nt];
    if (gq == 0) {
      float* pm = a.part_ml + (((int64_t)q * S + sp) * (HB * 16) + head0 + col) * 2;
      pm[0] = m;
      pm[1] = l;
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// A workgroup takes one query's 16-head block and 4 of its 32 accumulator
// tiles; a thread owns one accumulator slot (4 heads x 1 dim) and issues all
// of its partial loads (every split) before the first use.
__global__ __launch_bounds__(256) void k_attend_combine(AttendArgs a) {
  const int S = a.splits, H = a.heads, HB = (H + 15) / 16;
  const int q = blockIdx.x / (HB * 8), hb = (blockIdx.x / 8) % HB, ntg = blockIdx.x % 8;
  const int lane = threadIdx.x & 63, nt = ntg * 4 + (threadIdx.x >> 6);
  const int gq = lane >> 4, col = lane & 15;
  const int h0 = hb * 16 + 4 * gq;
  v4f os[kAttendMaxSplits];
  float ms[kAttendMaxSplits][4], ls[kAttendMaxSplits][4];
#pragma unroll
  for (int s = 0; s < kAttendMaxSplits; ++s) {
    os[s] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) { ms[s][i] = -__builtin_inff(); ls[s][i] = 0.0f; }
    if (s < S) {
      os[s] = *reinterpret_cast<const v4f*>(a.part_o + (((int64_t)q * S + s) * HB + hb) * (kLatent * 16) +
                                            (nt * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v2f ml = *reinterpret_cast<const v2f*>(a.part_ml + (((int64_t)q * S + s) * (HB * 16) + h0 + i) * 2);
        ms[s][i] = ml[0];
        ls[s][i] = ml[1];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float M = ms[0][i];
#pragma unroll
    for (int s = 1; s < kAttendMaxSplits; ++s) M = fmaxf(M, ms[s][i]);
    float den = 0.0f, acc = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int s = 0; s < kAttendMaxSplits; ++s) {
        const float wgt = ls[s][i] > 0.0f ? exp2f(ms[s][i] - M) : 0.0f;
        den += wgt * ls[s][i];
        acc += wgt * os[s][i];
      }
    }
    if (h0 + i >= H) continue;               // padding heads (H a multiple of 8)
    a.out[((int64_t)q * H + h0 + i) * kLatent + nt * 16 + col] = den > 0.0f ? acc / den : 0.0f;
    if (a.lse && nt == 0 && col == 0)
      a.lse[(int64_t)q * H + h0 + i] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attend, dim3((unsigned)(a.n_q * a.head_groups * a.splits)), dim3(kNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(k_attend_combine, dim3((unsigned)(a.n_q * ((a.heads + 15) / 16) * 8)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
