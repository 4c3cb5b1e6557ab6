// The Full scan's launch arguments and constants (kept apart from the other
// stages' so that a change elsewhere leaves the scan's sources untouched).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct ScanArgs {
  const uint8_t* idx_q;      // [n_q, Hi, d] fp8, or FP4 codes [n_q, Hi, d / 2]
  const float* idx_w;        // [n_q, Hi]
  const uint8_t* idx_k;      // [rows, d] fp8, or FP4 codes [rows, d / 2]
  // FP4 indexer rows (nullptr: fp8 rows): one E4M3 scale per 16 channels
  const uint8_t* idx_q_scales;   // [n_q, Hi, d / 16]
  const uint8_t* idx_k_scales;   // [rows, d / 16]
  const int64_t* seq_base;   // [n_q]
  const int32_t* n_visible;  // [n_q]
  int n_q, hi, d, swa, g;    // g: queries per sequence
  int tiles;                 // position tiles per query
  int tile_pos;              // positions per tile (multiple of 64)
  int tile_extra;            // tiles [0, tiles / 2) take tile_pos + tile_extra positions, the
                             // rest tile_pos - tile_extra (a multiple of 8; 0: equal tiles)
  int prefetch;              // LDS ring slots per wave (4, 6 or 8)
  int waves;                 // waves per workgroup (4 or 8)
  float* bscore;             // [n_q, ld]
  int64_t ld;
  // optional (nullptr: not written): the pool-select workspace, where each
  // tile stores the (min, max) order keys of its block scores at pair `tile`
  // and tile 0 clears the query's histogram
  uint32_t* pool_ws;
  int64_t pool_ws_stride;
  // paged keys (nullptr: position p of query q's sequence is row
  // seq_base[q] + p): row (pages[seq_base[q] + (p >> page_shift)] <<
  // page_shift) + (p mod 2^page_shift) of planes of `rows` rows
  const int32_t* pages;
  int page_shift;
  int64_t rows;
  // optional (nullptr: not written): every candidate position's score as an
  // order key, [n_q, ld_pkey] (position p of query q at q * ld_pkey + p; 0
  // for the positions past c in a query's last step), so that a Full layer's
  // Top-K can be selected without scoring the pool again
  uint32_t* pkey;
  int64_t ld_pkey;
  // optional (nullptr: not written): per group of kGroupBlocks consecutive
  // blocks of a query (128 positions), the largest of their block scores'
  // order keys, group i of query q at gkey[q * ld_gkey + i]; every tile then
  // starts at a multiple of 128 positions
  uint32_t* gkey;
  int64_t ld_gkey;
};

hipError_t launch_scan(const ScanArgs& a, hipStream_t s);

constexpr int kHistBins = 4096;        // pool histogram bins, cleared by the scan's tile 0
constexpr int kScanTile = 2048;        // default positions per scan workgroup
constexpr int kScanTileMin = 128;      // the smallest tile a small launch takes
constexpr int kScanSmallGrid = 64;     // launches of fewer workgroups take smaller tiles
constexpr int kScanPrefetch = 4;       // default LDS ring slots per wave
constexpr int kScanWaves = 4;          // default waves per scan workgroup
constexpr int kScanTileExtra = 512;    // uneven-tile shift when the grid is one round of two per CU
constexpr int kGroupBlocks = 16;       // blocks per group key

}  // namespace csa2
