// Expert MLPs as grouped matrix products on the gfx950 matrix cores (bf16
// inputs, fp32 sums), for batches where each expert sees many tokens, and the
// router's logits for such batches.
//
// Each expert is a SwiGLU MLP, hidden 5,120 -> intermediate 2,560 -> hidden
// ("Hugging Face releases Beam ..." MoE paragraph; "Reflection Releases Beam
// ...", section "Where Beam Saves and Where the Memory Bill Comes In"):
//   gate/up  h[slot, c] = silu(x[tok] . W_gu[e, c]) * (x[tok] . W_gu[e, I+c])
//   down     y[slot, n] = h[slot] . W_d[e, n]
//
// Work is the list of (expert, 256-slot M tile) entries built by the
// permutation kernels, crossed with 256-wide N tiles.  A gate/up N tile holds
// 128 gate rows of W_gu and the 128 matching up rows, so every wave owns both
// halves of its channels and applies silu(g)*u in registers; x rows are
// gathered by slot inside the A loads (no permuted copy of x).  Tiles move
// from global memory straight into LDS (global_load_lds_dwordx4), double
// buffered, 16-byte chunks XOR-swizzled by row so the MFMA operand reads are
// bank-conflict free; operand fragments are double buffered in registers.
// 8 waves (2 per SIMD) each compute 128x64 with 32x32x16 bf16 MFMA.
//
// Tile layout, DMA pattern and the XCD-aware tile order: grouped_tile.h.
//
// Router logits for many tokens use the same tile loop as a dense product:
// the fp32 router matrix is split exactly into three bf16 matrices, laid side
// by side along k (W3 [E, 3H]) and multiplied with x repeated three times
// (its column index wraps modulo H), so every product is exact and the sums
// are fp32.  The reduction is split into ks slices; the router's selection
// kernel adds the ks partial logits in a fixed order.
#include "grouped_tile.h"

namespace beam {
namespace {

using namespace tile;
constexpr int BK = 64;  // bf16 values per tile row per k-step

enum Mode { kGateUp = 0, kDown = 1 };

// acc[i][n] += A[arow_i] . B[brow_n] over columns [k0, k0 + nk*BK) of B,
// for the first NF of the wave's four 32-row A fragments (the others hold
// only padding rows past the tile's last valid row and are skipped).  A's
// column is the same index modulo a_period (a_period >= k0 + nk*BK when A is
// as wide as B).  a_off / b_off: this lane's element offsets (from a_base /
// b_base) of its kLoads A and B rows, chunk included; a_ok[i]: whether A row
// i is a valid row (padding rows are not loaded: their LDS rows only feed
// output rows that are never stored).  arow / brow: tile rows whose
// fragments this lane feeds to the MFMAs.  Ends with a barrier.
template <int NF>
__device__ __forceinline__ void tile_mainloop(
    const uint16_t* __restrict__ a_base, const uint32_t* a_off, const bool* a_ok,
    int a_period, const uint16_t* __restrict__ b_base, const uint32_t* b_off, int k0,
    int nk, TileLds& lds, f32x16 (&acc)[4][2], const int* arow, const int* brow) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto dma = [&](int buf, int k) {
    const int ka = k % a_period;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int region = wave + 8 * i;
      if (a_ok[i]) dma16(a_base + (a_off[i] + ka), &lds[buf][region * 1024]);
      dma16(b_base + (b_off[i] + k), &lds[buf][kTileBytes + region * 1024]);
    }
  };
  struct Frags {
    bf16x8 a[4], b[2];
  };
  auto load_frags = [&](Frags& f, int buf, int kk) {
    const int c = kk * 2 + lane / 32;
#pragma unroll
    for (int i = 0; i < NF; ++i)
      f.a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&lds[buf][swz(arow[i], c)]));
#pragma unroll
    for (int n = 0; n < 2; ++n)
      f.b[n] = as_bf16x8(*reinterpret_cast<const u32x4*>(&lds[buf][kTileBytes + swz(brow[n], c)]));
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[i][n] = mfma32x32x16(f.a[i], f.b[n], acc[i][n]);
  };
  // fragments of k16 step kk+1 are read while the 8 products of step kk run
  // (scheduling fences keep the compiler from folding the two fragment sets
  // into one and waiting on LDS before every product)
  auto compute = [&](int buf) {
    Frags f0, f1;
    load_frags(f0, buf, 0);
    load_frags(f1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(f0, buf, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(f1, buf, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
  };
  dma(0, k0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // buffer buf^1 was last read before the barrier that ended step kt-1
    if (kt + 1 < nk) dma(buf ^ 1, k0 + (kt + 1) * BK);
    if (NF > 0) compute(buf);
    __syncthreads();  // waits for this wave's loads, then for every wave
  }
}

// tile_mainloop with the wave's fragment count nf (0..4) made a constant.
__device__ __forceinline__ void tile_mainloop_rows(
    int nf, const uint16_t* __restrict__ a_base, const uint32_t* a_off, const bool* a_ok,
    int a_period, const uint16_t* __restrict__ b_base, const uint32_t* b_off, int k0,
    int nk, TileLds& lds, f32x16 (&acc)[4][2], const int* arow, const int* brow) {
  switch (nf) {
    case 4: tile_mainloop<4>(a_base, a_off, a_ok, a_period, b_base, b_off, k0, nk, lds, acc, arow, brow); break;
    case 3: tile_mainloop<3>(a_base, a_off, a_ok, a_period, b_base, b_off, k0, nk, lds, acc, arow, brow); break;
    case 2: tile_mainloop<2>(a_base, a_off, a_ok, a_period, b_base, b_off, k0, nk, lds, acc, arow, brow); break;
    case 1: tile_mainloop<1>(a_base, a_off, a_ok, a_period, b_base, b_off, k0, nk, lds, acc, arow, brow); break;
    default: tile_mainloop<0>(a_base, a_off, a_ok, a_period, b_base, b_off, k0, nk, lds, acc, arow, brow); break;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(
    const uint16_t* __restrict__ a_src,   // gate/up: x [T,H]; down: h [S,I]
    const uint16_t* __restrict__ w,       // W_gu [E,2I,H] or W_d [E,H,I]
    uint16_t* __restrict__ out,           // gate/up: h [S,I]; down: y [S,H]
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ meta, int E, int H, int I, int n_nt) {
  __shared__ __attribute__((aligned(16))) TileLds lds;

  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / 4, wn = wave % 4;

  // 32-bit element offsets from wave-uniform bases (the caller guarantees
  // S * max(H, I) < 2^31; one expert's weights are far below that).
  const uint16_t* wbase = (MODE == kGateUp) ? w + static_cast<int64_t>(e) * 2 * I * H
                                            : w + static_cast<int64_t>(e) * H * I;
  const int m_valid = min(BM, row_end - row0);
  uint32_t a_off[kLoads], b_off[kLoads];
  bool a_ok[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = dma_row(wave, lane, i);
    const int c = dma_chunk(r, lane);
    a_ok[i] = r < m_valid;
    int slot = row0 + r;
    if (slot > row_end - 1) slot = row_end - 1;  // padded rows: any valid row
    if (MODE == kGateUp) {
      a_off[i] = static_cast<uint32_t>(slot_token[slot]) * H + c * 8;
      // rows 0..127: gate channels nt*128 + r; rows 128..255: up channels
      const int wrow = (r < 128) ? (nt * 128 + r) : (I + nt * 128 + (r - 128));
      b_off[i] = static_cast<uint32_t>(wrow) * H + c * 8;
    } else {
      a_off[i] = static_cast<uint32_t>(slot) * I + c * 8;
      // the last N tile may run past H (H is a multiple of 128 only)
      b_off[i] = static_cast<uint32_t>(min(nt * BN + r, H - 1)) * I + c * 8;
    }
  }
  // A rows of this wave: wm*128 + mi*32 + lane%32.
  // B rows: gate/up -> gate wn*32 + lane%32 and up 128 + wn*32 + lane%32;
  //         down    -> wn*64 + ni*32 + lane%32.
  int arow[4], brow[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = wm * 128 + i * 32 + lane % 32;
#pragma unroll
  for (int n = 0; n < 2; ++n)
    brow[n] = (MODE == kGateUp) ? (n * 128 + wn * 32 + lane % 32)
                                : (wn * 64 + n * 32 + lane % 32);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};
  tile_mainloop_rows(wave_frags(m_valid, wm), a_src, a_off, a_ok, K, wbase, b_off, 0,
                     K / BK, lds, acc, arow, brow);

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      if (row >= row_end) continue;
      if (MODE == kGateUp) {
        const int ch = nt * 128 + wn * 32 + lane % 32;
        const float h = silu(acc[i][0][r]) * acc[i][1][r];
        out[static_cast<int64_t>(row) * I + ch] = f32_to_bf16_bits(h);
      } else {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = nt * BN + wn * 64 + n * 32 + lane % 32;
          if (col < H) out[static_cast<int64_t>(row) * H + col] = f32_to_bf16_bits(acc[i][n][r]);
        }
      }
    }
  }
}

// ---- 128- and 160-row tiles with a ring of three copy stages ----------------
// For batches whose experts hold few rows the products are bound by the
// weight bytes, and the 256-row tile's single stage in flight leaves HBM
// under-used.  These forms take 128 x 256 or 160 x 256 tiles with three 48 /
// 52 KiB stages (two in flight while one is consumed; 144 / 156 KiB of LDS).
// (A 64-row form with four 40 KiB stages measured no faster.)  A wave copies
// the same c = 4 + n_a regions every stage (n_a: its A regions, 8 rows each,
// that hold a valid row; rows past the last valid one inside such a region
// copy a valid row), so "stage s has landed" is a count of the wave's
// outstanding vector-memory operations: c times the stages issued after s
// (tile::ring_barrier).  8 waves:
// 2 along M (64 + 64 or 96 + 64 rows) x 4 along N, B rows as in the 256-row
// form.
namespace small {

template <int BMS>
struct Geo {
  static constexpr int kABytes = BMS * kRowBytes;
  static constexpr int kStage = kABytes + kTileBytes;
  static constexpr int kStages = 3;
  static constexpr int kRegions = BMS / 8;                     // 8-row A regions
  static constexpr int kALoads = (kRegions + 7) / 8;            // per wave: 2 or 3
  static constexpr int kBLoads = kTileBytes / (16 * kThreads);  // 4
  // rows of the waves with wm = 0 (the rest belong to wm = 1); a SIMD holds
  // one wave of each, so 160 rows split 96 + 64 still balance per SIMD
  static constexpr int kWaveRows = (BMS == 160) ? 96 : BMS / 2;
  static constexpr int kFrags = kWaveRows / 32;                 // wm = 0: 2 or 3
  static constexpr int kFrags1 = (BMS - kWaveRows) / 32;        // wm = 1: 2
};

template <int BMS, int NF>
__device__ __forceinline__ void ring_mainloop(
    const uint16_t* __restrict__ a_base, const uint32_t* a_off, const bool* a_ok, int c,
    const uint16_t* __restrict__ b_base, const uint32_t* b_off, int nk,
    unsigned char (&ring)[Geo<BMS>::kStages][Geo<BMS>::kStage],
    f32x16 (&acc)[Geo<BMS>::kFrags][2], const int* arow, const int* brow) {
  using G = Geo<BMS>;
  constexpr int S = G::kStages, P = S - 1;  // ring size, stages in flight
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto dma = [&](int st, int k) {
#pragma unroll
    for (int i = 0; i < G::kALoads; ++i)
      if (a_ok[i]) dma16(a_base + (a_off[i] + k), &ring[st][(wave + 8 * i) * 1024]);
#pragma unroll
    for (int i = 0; i < G::kBLoads; ++i)
      dma16(b_base + (b_off[i] + k), &ring[st][G::kABytes + (wave + 8 * i) * 1024]);
  };
  struct Frags {
    bf16x8 a[G::kFrags], b[2];
  };
  auto load_frags = [&](Frags& f, int st, int kk) {
    const int ch = kk * 2 + lane / 32;
#pragma unroll
    for (int i = 0; i < NF; ++i)
      f.a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&ring[st][swz(arow[i], ch)]));
#pragma unroll
    for (int n = 0; n < 2; ++n)
      f.b[n] = as_bf16x8(
          *reinterpret_cast<const u32x4*>(&ring[st][G::kABytes + swz(brow[n], ch)]));
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[i][n] = mfma32x32x16(f.a[i], f.b[n], acc[i][n]);
  };
  auto compute = [&](int st) {
    Frags f0, f1;
    load_frags(f0, st, 0);
    load_frags(f1, st, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(f0, st, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(f1, st, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
  };
#pragma unroll
  for (int s = 0; s < P; ++s)
    if (s < nk) dma(s, s * BK);
  ring_barrier(c * (min(P, nk) - 1));  // stage 0 landed
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt+P goes to the buffer last read in step kt-1 (ended by a barrier)
    const int kn = kt + P;
    if (kn < nk) dma(st == 0 ? S - 1 : st - 1, kn * BK);
    if (NF > 0) compute(st);
    ring_barrier(c * max(0, min(kn, nk - 1) - (kt + 1)));  // stage kt+1 landed
    st = (st == S - 1) ? 0 : st + 1;
  }
}

template <int BMS, int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_small(
    const uint16_t* __restrict__ a_src, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ out, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ meta, int E, int H,
    int I, int n_nt) {
  using G = Geo<BMS>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[G::kStages][G::kStage];
  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc, BMS)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / 4, wn = wave % 4;
  const uint16_t* wbase = (MODE == kGateUp) ? w + static_cast<int64_t>(e) * 2 * I * H
                                            : w + static_cast<int64_t>(e) * H * I;
  const int m_valid = min(BMS, row_end - row0);
  uint32_t a_off[G::kALoads], b_off[G::kBLoads];
  bool a_ok[G::kALoads];
  int c = G::kBLoads;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
#pragma unroll
  for (int i = 0; i < G::kALoads; ++i) {
    const int r = dma_row(wave, lane, i);
    // the region exists and its first row is valid
    a_ok[i] = uwave + 8 * i < G::kRegions && 8 * (uwave + 8 * i) < m_valid;
    c += a_ok[i];
    const int slot = min(row0 + r, row_end - 1);  // padding rows: a valid row
    a_off[i] = ((MODE == kGateUp) ? static_cast<uint32_t>(slot_token[slot]) * H
                                  : static_cast<uint32_t>(slot) * I) +
               dma_chunk(r, lane) * 8;
  }
#pragma unroll
  for (int i = 0; i < G::kBLoads; ++i) {
    const int r = dma_row(wave, lane, i);
    const int wrow = (MODE == kGateUp) ? ((r < 128) ? nt * 128 + r : I + nt * 128 + (r - 128))
                                       : min(nt * BN + r, H - 1);
    b_off[i] = static_cast<uint32_t>(wrow) * K + dma_chunk(r, lane) * 8;
  }
  int arow[G::kFrags], brow[2];
#pragma unroll
  for (int i = 0; i < G::kFrags; ++i) arow[i] = wm * G::kWaveRows + i * 32 + lane % 32;
#pragma unroll
  for (int n = 0; n < 2; ++n)
    brow[n] = (MODE == kGateUp) ? (n * 128 + wn * 32 + lane % 32)
                                : (wn * 64 + n * 32 + lane % 32);
  f32x16 acc[G::kFrags][2];
#pragma unroll
  for (int i = 0; i < G::kFrags; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};
  const int nf = min(wm == 0 ? G::kFrags : G::kFrags1,
                     max(0, (m_valid - wm * G::kWaveRows + 31) / 32));
  if (G::kFrags == 3 && nf == 3)
    ring_mainloop<BMS, 3>(a_src, a_off, a_ok, c, wbase, b_off, K / BK, ring, acc, arow, brow);
  else if (nf >= 2)
    ring_mainloop<BMS, 2>(a_src, a_off, a_ok, c, wbase, b_off, K / BK, ring, acc, arow, brow);
  else if (nf >= 1)
    ring_mainloop<BMS, 1>(a_src, a_off, a_ok, c, wbase, b_off, K / BK, ring, acc, arow, brow);
  else
    ring_mainloop<BMS, 0>(a_src, a_off, a_ok, c, wbase, b_off, K / BK, ring, acc, arow, brow);
#pragma unroll
  for (int i = 0; i < G::kFrags; ++i) {
    if (i >= nf) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + wm * G::kWaveRows + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      if (row >= row_end) continue;
      if (MODE == kGateUp) {
        const int ch = nt * 128 + wn * 32 + lane % 32;
        const float h = silu(acc[i][0][r]) * acc[i][1][r];
        out[static_cast<int64_t>(row) * I + ch] = f32_to_bf16_bits(h);
      } else {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = nt * BN + wn * 64 + n * 32 + lane % 32;
          if (col < H) out[static_cast<int64_t>(row) * H + col] = f32_to_bf16_bits(acc[i][n][r]);
        }
      }
    }
  }
}

}  // namespace small

// Router logits partials: part[z][t][e] = sum over k' in [z c, (z+1) c) of
// x[t, k' mod H] W3[e, k'] with c = 3H/ks (W3 [E, 3H] holds the three bf16
// terms of W_r one after another along k').  grid = ceil(T/256) * E/256 * ks.
__global__ __launch_bounds__(kThreads) void router_gemm_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w3,
    float* __restrict__ part, int T, int E, int H, int ks) {
  __shared__ __attribute__((aligned(16))) TileLds lds;
  const int n_nt = E / BN;
  const int per_m = n_nt * ks;
  const int mt = blockIdx.x / per_m;
  const int nt = (blockIdx.x % per_m) / ks;
  const int z = blockIdx.x % ks;
  const int row0 = mt * BM;
  const int kc = 3 * H / ks;

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / 4, wn = wave % 4;
  const int m_valid = min(BM, T - row0);
  uint32_t a_off[kLoads], b_off[kLoads];
  bool a_ok[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = dma_row(wave, lane, i);
    const int c = dma_chunk(r, lane);
    a_ok[i] = r < m_valid;
    const int t = min(row0 + r, T - 1);  // padded rows: any valid row
    a_off[i] = static_cast<uint32_t>(t) * H + c * 8;
    b_off[i] = static_cast<uint32_t>(nt * BN + r) * (3 * H) + c * 8;
  }
  int arow[4], brow[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = wm * 128 + i * 32 + lane % 32;
#pragma unroll
  for (int n = 0; n < 2; ++n) brow[n] = wn * 64 + n * 32 + lane % 32;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};
  tile_mainloop_rows(wave_frags(m_valid, wm), x, a_off, a_ok, H, w3, b_off, z * kc,
                     kc / BK, lds, acc, arow, brow);

  float* dst = part + static_cast<int64_t>(z) * T * E + nt * BN;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = row0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      if (t >= T) continue;
#pragma unroll
      for (int n = 0; n < 2; ++n)
        dst[static_cast<int64_t>(t) * E + wn * 64 + n * 32 + lane % 32] = acc[i][n][r];
    }
}

}  // namespace

hipError_t launch_router_gemm(const Plan& p, const void* x, const uint16_t* w3,
                              float* part, hipStream_t s, Timer* tm) {
  const int n_nt = p.E / BN;
  const unsigned grid = static_cast<unsigned>(ceil_div(p.T, BM) * n_nt * p.ks);
  BEAM_LAUNCH(tm, "router_gemm_bf16", router_gemm_bf16, dim3(grid), dim3(kThreads), 0, s,
              static_cast<const uint16_t*>(x), w3, part, static_cast<int>(p.T), p.E, p.H,
              p.ks);
  return hipGetLastError();
}

hipError_t launch_grouped_bf16(const Plan& p, const void* x,
                               const void* w_gate_up, const void* w_down,
                               void* ws, hipStream_t s, Timer* tm) {
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* toff = ws_at<int32_t>(ws, p.off_tile_off);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  uint16_t* h = ws_at<uint16_t>(ws, p.off_h);
  uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
  const int nt_gu = p.I / 128;
  const int nt_dn = static_cast<int>(ceil_div(p.H, BN));
#define BEAM_SMALL_TILES(BMS)                                                                \
  BEAM_LAUNCH(tm, "grouped_gate_up_bf16", (small::grouped_gemm_bf16_small<BMS, kGateUp>),    \
              grid_for(p, nt_gu), dim3(kThreads), 0, s, static_cast<const uint16_t*>(x),      \
              static_cast<const uint16_t*>(w_gate_up), h, slot_token, counts, offsets, toff,  \
              meta, p.E, p.H, p.I, nt_gu);                                                    \
  BEAM_LAUNCH(tm, "grouped_down_bf16", (small::grouped_gemm_bf16_small<BMS, kDown>),         \
              grid_for(p, nt_dn), dim3(kThreads), 0, s, h,                                    \
              static_cast<const uint16_t*>(w_down), y, slot_token, counts, offsets, toff,     \
              meta, p.E, p.H, p.I, nt_dn);                                                    \
  return hipGetLastError()
  if (p.bm == 128) { BEAM_SMALL_TILES(128); }
  if (p.bm == 160) { BEAM_SMALL_TILES(160); }
#undef BEAM_SMALL_TILES
  BEAM_LAUNCH(tm, "grouped_gate_up_bf16", grouped_gemm_bf16<kGateUp>, grid_for(p, nt_gu),
              dim3(kThreads), 0, s, static_cast<const uint16_t*>(x),
              static_cast<const uint16_t*>(w_gate_up), h, slot_token, counts,
              offsets, toff, meta, p.E, p.H, p.I, nt_gu);
  BEAM_LAUNCH(tm, "grouped_down_bf16", grouped_gemm_bf16<kDown>, grid_for(p, nt_dn),
              dim3(kThreads), 0, s, h, static_cast<const uint16_t*>(w_down), y,
              slot_token, counts, offsets, toff, meta, p.E, p.H, p.I, nt_dn);
  return hipGetLastError();
}

}  // namespace beam
