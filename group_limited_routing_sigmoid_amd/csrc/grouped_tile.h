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
constexpr int kBandM = 4;                   // M tiles per band of the logical order
constexpr int kQuadN = 8;                   // N tiles per quad
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

struct Coords {
  int e;        // expert
  int nt;       // N tile
  int row0;     // first slot of the M tile
  int row_end;  // first slot past the expert's slots
};

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, and
// start roughly in order.  The logical tiles form two sequences: those of
// hot experts (several M tiles, weights reused) and those of cold experts
// (one tile, weights streamed once from HBM); inside a sequence the order is
// expert, then bands of band_m M tiles (default 4), then quads of quad_n N
// tiles (default 8), the M tile moving fastest inside a quad.  The
// sequences are cut into chunks of 32 tiles, and chunk
// g = 8 (b / 256) + b % 8 goes to workgroups b of one
// round of 256 (one tile per compute unit) on one XCD: chunk g is cold when
// floor((g + 1) C / N) > floor(g C / N) (C cold chunks of N), so cold chunks
// are spread evenly over the rounds.  Then
// - the hot chunks of a round are consecutive: the XCDs on them share one
//   window of one expert's weights and token rows in the last-level cache,
//   and each XCD's 32 tiles (about 4 M x 8 N) share operand slices in its L2
//   (measured on the 16K-token layer: gate/up 8.20 -> 7.53 ms against XCDs
//   walking separate eighths of an expert-major order; with the four-wave
//   bf16 kernels 4 M x 8 N measured about 1% faster than 8 M x 4 N, gate/up
//   and down, on the 16K-token and expert-parallel layers, while 16 x 2,
//   2 x 16 and 2 x 10 were slower; the 4-bit path keeps 8 M x 4 N);
// - the cold chunks stream weights from HBM while the hot ones keep the
//   matrix cores busy, instead of the chip alternating between the two.
// Returns false for workgroups past the last tile.
__device__ __forceinline__ bool tile_coords(const int32_t* counts, const int32_t* offsets,
                                            const int32_t* tt, const int32_t* meta,
                                            int E, int n_nt, Coords& c, int bm = BM,
                                            int band_m = kBandM, int quad_n = kQuadN) {
  const int nm = meta[kMetaTiles], nmh = meta[kMetaHot];
  const int nh = nmh * n_nt, nc = (nm - nmh) * n_nt;  // logical tiles per sequence
  const int chh = (nh + kXcdRun - 1) / kXcdRun, chc = (nc + kXcdRun - 1) / kXcdRun;
  const int ch = chh + chc;
  const int b = blockIdx.x;
  const int g = (b / kRound) * kXcds + b % kXcds;
  if (g >= ch) return false;
  const int c0 = static_cast<int>(static_cast<int64_t>(g) * chc / ch);
  const int c1 = static_cast<int>(static_cast<int64_t>(g + 1) * chc / ch);
  const bool cold = c1 > c0;
  const int L = (cold ? c0 : g - c0) * kXcdRun + (b / kXcds) % kXcdRun;
  if (L >= (cold ? nc : nh)) return false;
  const int mbase = cold ? nmh : 0;  // the sequence's first M tile
  const int e = tt[tt_expert(E) + mbase + L / n_nt];
  const int t0 = tt[e] - mbase, nt_e = tt[tt_count(E) + e];
  const int j = L - t0 * n_nt;
  const int band = j / (band_m * n_nt);
  const int gm = min(band_m, nt_e - band * band_m);
  const int jj = j - band * band_m * n_nt;
  const int q = jj / (gm * quad_n);
  const int rem = jj - q * gm * quad_n;  // the last quad may be narrower
  c.e = e;
  c.nt = q * quad_n + rem / gm;
  c.row0 = offsets[e] + (band * band_m + rem % gm) * bm;
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

// Grid of a grouped launch: whole rounds covering an upper bound on the
// chunks (each of the two sequences may end in a partial chunk).
inline dim3 grid_for(const Plan& p, int n_nt) {
  const int64_t chunks = ceil_div(p.max_tiles * n_nt, kXcdRun) + 1;
  return dim3(static_cast<unsigned>(ceil_div(chunks, kXcds) * kRound));
}

}  // namespace tile
}  // namespace beam
