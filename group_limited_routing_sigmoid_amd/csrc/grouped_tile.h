// Tile machinery shared by the grouped expert GEMMs (bf16 and e4m3): the
// LDS tile layout, its global -> LDS copy pattern and the XCD-aware mapping
// of workgroups to (expert, M tile, N tile).
//
// A tile is 256 rows of 128 bytes (64 bf16 or 128 e4m3 values along k), so
// both GEMMs stage the same bytes per k-step and share every address below.
#pragma once

#include "common.h"
#include "internal.h"

namespace beam {
namespace tile {

constexpr int BM = kGemmBM;                 // 256 rows (slots) per M tile
constexpr int BN = 256;                     // weight rows per N tile
constexpr int kThreads = 512;               // 8 waves
constexpr int kRowBytes = 128;              // bytes per tile row per k-step
constexpr int kTileBytes = BM * kRowBytes;  // 32 KiB per operand tile
constexpr int kXcds = 8;
constexpr int kXcdRun = 32;                 // consecutive logical tiles per XCD per round
constexpr int kRound = kXcds * kXcdRun;     // logical tiles per round
constexpr int kBandM = 8;                   // M tiles per band of the logical order
constexpr int kQuadN = 4;                   // N tiles per quad
constexpr int kLoads = kTileBytes / (16 * kThreads);  // DMA regions per wave per operand

// Two stages of (A tile, B tile).
typedef unsigned char TileLds[2][2 * kTileBytes];

__device__ __forceinline__ int swz(int row, int chunk) {
  // the 8 chunks of any 8 consecutive rows land on distinct bank groups,
  // and so do the even (and the odd) rows of any 16 consecutive rows
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Tile row and logical 16-byte chunk that lane `lane` of wave `wave` loads in
// DMA region i: one region = 1 KiB = 8 tile rows, lane l writing physical
// chunk l % 8 of row l / 8; wave w fills regions w + 8i.
__device__ __forceinline__ int dma_row(int wave, int lane, int i) {
  return 8 * (wave + 8 * i) + lane / 8;
}
__device__ __forceinline__ int dma_chunk(int row, int lane) {
  return (lane % 8) ^ ((row ^ (row >> 3)) & 7);
}

// Largest e with tile_off[e] * n_nt <= L (tile_off is non-decreasing).
__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int n_nt, int L) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] * n_nt <= L) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct Coords {
  int e;        // expert
  int nt;       // N tile
  int row0;     // first slot of the M tile
  int row_end;  // first slot past the expert's slots
};

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, and
// start roughly in order.  Workgroup b takes logical tile
//   256 (b / 256) + 32 (b % 8) + (b / 8) % 32,
// so the chip works through the logical order in rounds of 256 tiles (one
// tile per compute unit), every XCD taking 32 consecutive ones.  The logical
// order is: expert, then bands of 8 M tiles, then quads of 4 N tiles, with
// the M tile moving fastest inside a quad.  At any time the 8 XCDs then
// share one window of one expert's weights and token rows in the last-level
// cache, and each XCD's 32 tiles are about 8 M x 4 N tiles whose operand
// slices its L2 shares (measured on the 16K-token layer: gate/up 8.20 ->
// 7.53 ms against XCDs walking separate eighths of the order; the blocking
// alone, without the shared window, gained nothing).
// Returns false for workgroups past the last logical tile.
__device__ __forceinline__ bool tile_coords(const int32_t* counts, const int32_t* offsets,
                                            const int32_t* tile_off, const int32_t* meta,
                                            int E, int n_nt, Coords& c, int bm = BM) {
  const int n_log = meta[kMetaTiles] * n_nt;
  const int b = blockIdx.x;
  const int L = (b / kRound) * kRound + (b % kXcds) * kXcdRun + (b / kXcds) % kXcdRun;
  if (L >= n_log) return false;
  const int e = find_expert(tile_off, E, n_nt, L);
  const int t0 = tile_off[e], nt_e = tile_off[e + 1] - t0;
  const int j = L - t0 * n_nt;
  const int band = j / (kBandM * n_nt);
  const int gm = min(kBandM, nt_e - band * kBandM);
  const int jj = j - band * kBandM * n_nt;
  const int q = jj / (gm * kQuadN);
  const int rem = jj - q * gm * kQuadN;  // the last quad may be narrower
  c.e = e;
  c.nt = q * kQuadN + rem / gm;
  c.row0 = offsets[e] + (band * kBandM + rem % gm) * bm;
  c.row_end = offsets[e] + counts[e];
  return true;
}

// Number of a wave's 32-row A fragments (rows wm*128 + 32 i ...) that hold
// at least one of the tile's m_valid rows.
__device__ __forceinline__ int wave_frags(int m_valid, int wm) {
  return min(4, max(0, (m_valid - wm * 128 + 31) / 32));
}

// Copy rings: wait until at most n (0..15, wave-uniform) of this wave's
// vector-memory operations are outstanding and its LDS reads are done, then
// meet every wave.  Loads complete in issue order, so after a wave has issued
// the copies of the stages after s, "stage s has landed" is n = the number of
// those later copies.  Any other n waits for all (always safe).
#define BEAM_RING_BARRIER(n) \
  asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")
__device__ __forceinline__ void ring_barrier(int n) {
  switch (n) {
    case 1: BEAM_RING_BARRIER(1); break;
    case 2: BEAM_RING_BARRIER(2); break;
    case 3: BEAM_RING_BARRIER(3); break;
    case 4: BEAM_RING_BARRIER(4); break;
    case 5: BEAM_RING_BARRIER(5); break;
    case 6: BEAM_RING_BARRIER(6); break;
    case 7: BEAM_RING_BARRIER(7); break;
    case 8: BEAM_RING_BARRIER(8); break;
    case 9: BEAM_RING_BARRIER(9); break;
    case 10: BEAM_RING_BARRIER(10); break;
    case 11: BEAM_RING_BARRIER(11); break;
    case 12: BEAM_RING_BARRIER(12); break;
    case 13: BEAM_RING_BARRIER(13); break;
    case 14: BEAM_RING_BARRIER(14); break;
    case 15: BEAM_RING_BARRIER(15); break;
    default: BEAM_RING_BARRIER(0); break;
  }
}
#undef BEAM_RING_BARRIER

// Grid of a grouped launch: an upper bound on the logical tiles, rounded to
// whole rounds (the workgroup -> tile map is a bijection on each round).
inline dim3 grid_for(const Plan& p, int n_nt) {
  const int64_t rounds = ceil_div(p.max_tiles * n_nt, kRound);
  return dim3(static_cast<unsigned>(rounds * kRound));
}

}  // namespace tile
}  // namespace beam
