// 4-bit expert weights: OCP MX FP4 (E2M1 codes, two per byte, the even k in
// the low nibble) with one E8M0 scale per 32 consecutive k of a weight row,
// and activations quantised on the fly to MXFP8 (E4M3 codes, one E8M0 scale
// per 32 channels, the scale the smallest power of two that keeps the
// block's largest value within 448).  The pages ship a 4-bit checkpoint for other hardware
// ("Hugging Face releases Beam ..." checkpoint paragraph; "Reflection Beam",
// section "Where to run it"); MX is the 4-bit format the gfx950 matrix cores
// scale in hardware: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies each lane's
// 32 k-values by 2^(scale - 127) for both operands, so the block scales are
// exact and no vector work rescales the sums.
//
// Two expert paths: grouped tiles with copy rings (the default at every batch
// size; measured ahead of streaming down to one token) and weight-streaming
// kernels (on request).  Streaming: weights are the 32-row A side (fp4), up
// to 32 tokens the B side (fp8).  Gate/up: a wave owns 16 gate
// and the 16 matching up rows, whose products land in the same lane (rows r
// and r + 16 are accumulator elements q and q + 8).  Down: a wave owns 32
// rows of W_d.  Experts with more than 32 tokens are handled in chunks.
#include <type_traits>

#include "grouped_tile.h"

namespace beam {
namespace {

// Exponent of an activation block: the smallest power of two 2^x with
// amax / 2^x <= 448 (the largest E4M3 value), so the block maximum never
// saturates; clamped to the E8M0 range [-127, 127], -127 for a zero block.
// floor(log2(amax)) - 8 puts amax / 2^x in [256, 512); one more when above 448.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int eb = (__float_as_uint(amax) >> 23) & 0xFF;  // amax >= 0
  const int fl = (eb == 0) ? -127 : eb - 127;            // floor(log2), subnormals clamp
  int x = max(-127, min(127, fl - 8));
  if (amax > 0.0f && x < 127 && ldexpf(amax, -x) > 448.0f) ++x;
  return x;
}

// One thread per 32-value block of a row: E4M3 codes of v * 2^-x (exact
// scaling, round to nearest even; |v * 2^-x| <= 448 by the choice of x) and
// the E8M0 code x + 127.  With slot_of (x in the grouped forward) the four
// codes of each 128-column block kb also go, as one word, to the K slots of
// the row: word kb * S + slot, so that a tile stage of the grouped products
// reads its rows' words as one run rather than one cache line per row.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_mxfp8_rows(
    const void* __restrict__ v, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales, const int32_t* __restrict__ slot_of, int K,
    uint8_t* __restrict__ xss, int S) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbc = cols / 32;
  // cols % 128 == 0: the lanes that return are whole groups of four
  if (blk >= rows * nbc) return;
  const int64_t at = (blk / nbc) * cols + (blk % nbc) * 32;
  float a[32];
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = ld16(static_cast<const uint16_t*>(v) + at + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        a[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 w = ld16(static_cast<const float*>(v) + at + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[4 * i + j] = __uint_as_float(w[j]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(a[i]));
  const int x = mx8_exponent(amax);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i / 4][i % 4] = e4m3x4(ldexpf(a[4 * i], -x), ldexpf(a[4 * i + 1], -x),
                               ldexpf(a[4 * i + 2], -x), ldexpf(a[4 * i + 3], -x));
  }
  st16(q + at, out[0]);
  st16(q + at + 16, out[1]);
  const uint32_t b = static_cast<uint32_t>(x + 127);
  scales[blk] = static_cast<uint8_t>(b);
  if (xss) {
    // the four scale bytes of a 128-column block come from four consecutive
    // lanes; the word goes to every slot of the row, block-major
    const int l0 = (threadIdx.x % kWave) & ~3;
    const uint32_t word = __shfl(b, l0) | (__shfl(b, l0 + 1) << 8) |
                          (__shfl(b, l0 + 2) << 16) | (__shfl(b, l0 + 3) << 24);
    if (threadIdx.x % 4 == 0) {
      const int64_t row = blk / nbc, kb = (blk % nbc) / 4;
      for (int k = 0; k < K; ++k)
        reinterpret_cast<uint32_t*>(xss)[kb * S + slot_of[row * K + k]] = word;
    }
  }
}

// D = A(32x64, E2M1) * B(64x32, E4M3) + C with per-lane E8M0 scales.  Lane
// l = 32 h + r supplies row r of A and column r of B.  With E2M1 A (4
// registers) the matrix cores read the lane's 32 nibbles as k = 16 h + j
// (j < 16) and 32 + 16 h + (j - 16), and apply the lane's A scale to exactly
// those; the B scale of lane l covers the same k positions of column r.  So
// a lane hands over one contiguous 32-value weight block (bytes 16 h .. of
// the 32-byte step) with its scale, and its B side is activation values
// 16 h .. 16 h + 15 and 32 + 16 h .. 32 + 16 h + 15 of the 64-value step
// (the same k positions) with the scale of activation block h; every
// product then carries its own two block scales.
__device__ __forceinline__ f32x16 mfma_mx(u32x4 a, u32x4 b0, u32x4 b1, f32x16 c, uint32_t sa,
                                          uint32_t sb) {
  const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                    (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

constexpr int kThreads = 256;
constexpr int kWaves = 4;
#ifndef BEAM_MX_UNROLL
#define BEAM_MX_UNROLL 8
#endif
constexpr int kMxUnroll = BEAM_MX_UNROLL;  // 64-deep k-steps in flight per wave
static_assert(kMxUnroll % 2 == 0, "scale words cover two k-steps");

// byte b of a little-endian array of words
__device__ __forceinline__ uint32_t byte_of(const uint32_t* w, int b) {
  return (w[b / 4] >> (8 * (b % 4))) & 0xFFu;
}

// Streams `rows32` (32 weight rows of n_k 64-deep steps, at w_row / s_row for
// this lane's row) against the chunk's tokens: returns the 32x32 sums.
// Lane l: weight row l % 32, token column l % 32 (valid if has_tok).
__device__ __forceinline__ f32x16 mx_rows(const uint8_t* __restrict__ w_row,
                                          const uint8_t* __restrict__ s_row,
                                          const uint8_t* __restrict__ a_row,
                                          const uint8_t* __restrict__ as_row, bool has_tok,
                                          int n_k, int half) {
  f32x16 acc0 = {}, acc1 = {};
  for (int s0 = 0; s0 < n_k; s0 += kMxUnroll) {
    u32x4 wv[kMxUnroll], xv[kMxUnroll][2];
    uint32_t ws[kMxUnroll / 2], xs[kMxUnroll / 2];
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const bool in = s0 + u < n_k;
      wv[u] = in ? ld16(w_row + (s0 + u) * 32 + half * 16) : u32x4{0, 0, 0, 0};
      xv[u][0] = (in && has_tok) ? ld16(a_row + (s0 + u) * 64 + half * 16) : u32x4{0, 0, 0, 0};
      xv[u][1] = (in && has_tok) ? ld16(a_row + (s0 + u) * 64 + 32 + half * 16) : u32x4{0, 0, 0, 0};
    }
    // scale bytes of steps s0 .. s0+U-1: 2 per step (the two 32-value halves)
#pragma unroll
    for (int i = 0; i < kMxUnroll / 2; ++i) {
      const bool in = s0 + 2 * i < n_k;
      ws[i] = in ? *reinterpret_cast<const uint32_t*>(s_row + 2 * s0 + 4 * i) : 127u;
      xs[i] = (in && has_tok) ? *reinterpret_cast<const uint32_t*>(as_row + 2 * s0 + 4 * i)
                              : 0x7F7F7F7Fu;
    }
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const uint32_t sa = byte_of(ws, 2 * u + half), sb = byte_of(xs, 2 * u + half);
      if (u % 2 == 0) acc0 = mfma_mx(wv[u], xv[u][0], xv[u][1], acc0, sa, sb);
      else            acc1 = mfma_mx(wv[u], xv[u][0], xv[u][1], acc1, sa, sb);
    }
  }
  return acc0 + acc1;
}

// Gate/up: one wave per (active expert j, 16-channel block); rows 0..15 of
// its A side are gate channels cb*16 + r, rows 16..31 the up channels.
// grid ceil(max_active * I/16 / 4), block 256.
__global__ __launch_bounds__(kThreads) void stream_gate_up_mx(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, float* __restrict__ h,
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ meta, int H, int I) {
  const int n_cb = I / 16;
  const int item = blockIdx.x * kWaves + threadIdx.x / kWave;
  const int j = item / n_cb, cb = item % n_cb;
  if (j >= meta[kMetaActive]) return;
  const int e = active[j];
  const int off = offsets[e], cnt = counts[e];
  const int lane = threadIdx.x % kWave, r = lane % 32, half = lane / 32;
  const int wrow = (r < 16) ? (cb * 16 + r) : (I + cb * 16 + (r - 16));
  const int64_t grow = static_cast<int64_t>(e) * 2 * I + wrow;
  const uint8_t* w_row = w + grow * (H / 2);
  const uint8_t* s_row = ws + grow * (H / 32);
  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const bool has_tok = r < cnt - c0;
    const int64_t tok = has_tok ? slot_token[off + c0 + r] : 0;
    const f32x16 acc = mx_rows(w_row, s_row, xq + tok * H, xs + tok * (H / 32), has_tok, H / 64,
                               half);
    if (has_tok) {
      // element q: row 8*(q/4) + 4*half + q%4 (q < 8: gate), up row + 16 in q + 8
      float* hr = h + static_cast<int64_t>(off + c0 + r) * I + cb * 16;
#pragma unroll
      for (int q = 0; q < 8; ++q) hr[8 * (q / 4) + 4 * half + q % 4] = silu(acc[q]) * acc[q + 8];
    }
  }
}

// Down: one wave per (active expert j, 32 rows of W_d); the tokens' h in
// MXFP8.  grid ceil(max_active * H/32 / 4), block 256.
__global__ __launch_bounds__(kThreads) void stream_down_mx(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, float* __restrict__ y,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ meta, int H, int I) {
  const int n_ob = H / 32;
  const int item = blockIdx.x * kWaves + threadIdx.x / kWave;
  const int j = item / n_ob, ob = item % n_ob;
  if (j >= meta[kMetaActive]) return;
  const int e = active[j];
  const int off = offsets[e], cnt = counts[e];
  const int lane = threadIdx.x % kWave, r = lane % 32, half = lane / 32;
  const int64_t grow = static_cast<int64_t>(e) * H + ob * 32 + r;
  const uint8_t* w_row = w + grow * (I / 2);
  const uint8_t* s_row = ws + grow * (I / 32);
  for (int c0 = 0; c0 < cnt; c0 += 32) {
    const bool has_tok = r < cnt - c0;
    const int64_t slot = off + c0 + (has_tok ? r : 0);
    const f32x16 acc = mx_rows(w_row, s_row, hq + slot * I, hs + slot * (I / 32), has_tok,
                               I / 64, half);
    if (has_tok) {
      float* yr = y + static_cast<int64_t>(off + c0 + r) * H + ob * 32;
#pragma unroll
      for (int q = 0; q < 16; ++q) yr[8 * (q / 4) + 4 * half + q % 4] = acc[q];
    }
  }
}


// ---- grouped E2M1 x E4M3 GEMM -----------------------------------------------
// Same work list and XCD order as the bf16 grouped GEMM (M tiles of BMS = 256
// or 128 slots x 256-row N tiles), 128 k per stage, stages copied straight
// into LDS: activation tile (E4M3, BMS slots x 128 bytes, the bf16 tiles'
// layout and swizzle), weight tile (E2M1, 256 rows x 64 bytes), and both
// tiles' E8M0 bytes (4 per row per stage: the activations' from words kept
// per slot and block-major, one run per stage; the weights' in the stage or,
// when K % 512 == 0, in periods of four stages, below).  The stages form a ring (2 or 3
// of 50 KiB for 256 slots, 4 of 33.5 KiB for 128): the copies of all but the
// stage being consumed are in flight, and a wave copies the same number of
// regions every stage, so each wait is a count of its outstanding copies
// (tile::ring_barrier).  The weights are the MFMA A side, the slots the B
// side, so a wave's accumulators are channels x slots; a wave owns 32
// channels x BMS/2 slots twice (gate and the matching up channels for
// gate/up, 64 consecutive output columns for down).
namespace mxg {

using namespace tile;

// With two stages (256 slots) an expert's last tile may hold 32 extension
// slots past the 256: their activation rows and scale words get an area of
// their own after each stage's tiles.
constexpr int kXtRows = 32;
// PER (K a multiple of 512): the weight tile's E8M0 bytes do not travel in
// the stages, 4 bytes of each of its 256 rows per stage (256 scattered
// cache lines for 1 KiB), but in periods of kPer stages: 16 bytes of a row,
// a quarter of the rows with each stage, into a ring of kPerSlots period
// buffers after the stages (row-major, 16 bytes per row).
constexpr int kPer = 4;
constexpr int kPerSlots = 3;
template <int BMS, int STAGES, bool PER>
struct Geo {
  static constexpr int kXBytes = BMS * 128;  // activation tile per stage
  static constexpr int kWBytes = BN * 64;    // weight tile per stage
  static constexpr int kXtOff = kXBytes + kWBytes + (BMS + (PER ? 0 : BN)) * 4;
  static constexpr bool kExt = STAGES == 2;  // room for extension slots
  static constexpr int kStage = kXtOff + (kExt ? kXtRows * 128 + 256 : 0);
  static constexpr int kStages = STAGES;
  static constexpr int kPerBytes = PER ? kPerSlots * BN * 16 : 0;
  static constexpr int kXLoads = kXBytes / (16 * tile::kThreads);  // 4 or 2
  static constexpr int kXsWaves = BMS / 64;  // waves copying activation scale words
  static constexpr int kJ = BMS / 64;        // 32-slot fragments per wave
};

__device__ __forceinline__ int wswz(int row, int chunk) {  // 64-byte weight rows
  return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

enum Mode { kGateUp = 0, kDown = 1 };

// XT: also the extension slots (B rows of the extension area) against the
// wave's A fragment wm into accx (gate channels for wm = 0, up channels for
// wm = 1 on gate/up; output columns wn*64 + wm*32 .. on down).  WS: the
// stage's scale word of weight row t at WS[t * (PER ? 4 : 1)].
template <int BMS, int NJ, bool XT, bool PER>
__device__ __forceinline__ void stage_products(const unsigned char* st, const uint32_t* WS,
                                               f32x16 (&acc)[2][BMS / 64], f32x16& accx,
                                               const int* wrow, const int* srow, int half,
                                               int wm) {
  using G = Geo<BMS, 2, PER>;
  const unsigned char* X = st;
  const unsigned char* W = st + G::kXBytes;
  const uint32_t* XS = reinterpret_cast<const uint32_t*>(st + G::kXBytes + G::kWBytes);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 a[2];
    uint32_t sa[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      a[f] = *reinterpret_cast<const u32x4*>(W + wswz(wrow[f], 2 * ks + half));
      sa[f] = (WS[wrow[f] * (PER ? 4 : 1)] >> (8 * (2 * ks + half))) & 0xFFu;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = srow[j];
      const int key = (row ^ (row >> 3)) & 7;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(X + row * 128 + (((4 * ks + half) ^ key) << 4));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(X + row * 128 + (((4 * ks + 2 + half) ^ key) << 4));
      const uint32_t sb = (XS[row] >> (8 * (2 * ks + half))) & 0xFFu;
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[f][j] = mfma_mx(a[f], b0, b1, acc[f][j], sa[f], sb);
    }
    if (XT) {
      const unsigned char* XX = st + G::kXtOff;
      const uint32_t* XXS = reinterpret_cast<const uint32_t*>(XX + kXtRows * 128);
      const int row = srow[0] % 32;  // the lane's extension slot
      const int key = (row ^ (row >> 3)) & 7;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(XX + row * 128 + (((4 * ks + half) ^ key) << 4));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(XX + row * 128 + (((4 * ks + 2 + half) ^ key) << 4));
      const uint32_t sb = (XXS[row] >> (8 * (2 * ks + half))) & 0xFFu;
      accx = mfma_mx(wm ? a[1] : a[0], b0, b1, accx, wm ? sa[1] : sa[0], sb);
    }
  }
}

template <int BMS, int STAGES, int MODE, bool PER>
__global__ __launch_bounds__(tile::kThreads) void grouped_gemm_mx(
    const uint8_t* __restrict__ xq,      // gate/up: xq [T,H]; down: hq [S,I]  (E4M3)
    const uint8_t* __restrict__ xs,      // their E8M0 bytes per slot: [K/128][S] words
    const uint8_t* __restrict__ w,       // W_gu [E,2I,H/2] or W_d [E,H,I/2] (E2M1 pairs)
    const uint8_t* __restrict__ ws,      // [E,2I,H/32] or [E,H,I/32]
    void* __restrict__ out,              // gate/up: hq [S,I] (E4M3); down: y [S,H] (fp32)
    uint8_t* __restrict__ out_scale,     // gate/up: hs [I/128][S] words (E8M0); down: unused
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ meta, int E, int H, int I, int n_nt, int xt, int n_slots) {
  using G = Geo<BMS, STAGES, PER>;
  constexpr int S = G::kStages, P = S - 1;  // ring size, stages in flight
  // the stages, then (PER) the period buffers: one object, so the compiler
  // sees the copies and the reads of both as one array
  __shared__ __attribute__((aligned(16))) unsigned char lds[S * G::kStage + G::kPerBytes];
  constexpr int kPerOff = S * G::kStage;
  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc, BMS, 8, 4)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int nk = K / 128;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int wm = wave / 4, wn = wave % 4, r = lane % 32, half = lane / 32;
  const int m_valid = min(BMS, row_end - row0);
  // extension slots: only in an expert's last tile, when tiles may extend
  const int m_all = row_end - row0;
  const int x_rows = (G::kExt && m_all > BMS && m_all <= BMS + xt) ? m_all - BMS : 0;
  const int64_t nrows = (MODE == kGateUp) ? 2 * I : H;
  const uint8_t* wb = w + static_cast<int64_t>(e) * nrows * (K / 2);
  const uint8_t* wsb = ws + static_cast<int64_t>(e) * nrows * (K / 32);
  auto wrow_of = [&](int t) {  // weight row of tile row t
    return (MODE == kGateUp) ? ((t < 128) ? nt * 128 + t : I + nt * 128 + (t - 128))
                             : min(nt * BN + t, H - 1);
  };
  auto slot_src = [&](int t) {  // activation row of tile row t (padded rows: a valid one)
    const int slot = min(row0 + t, row_end - 1);
    return (MODE == kGateUp) ? slot_token[slot] : slot;
  };
  // copy sources: activations kXLoads x 1 KiB regions per wave (8 rows of
  // 128 B; regions whose first row is padding are not copied), weights
  // 2 x 1 KiB (16 rows of 64 B); scale words: waves 0 .. kXsWaves-1 the
  // activation rows 64 w + lane, the next 4 waves the weight rows
  uint32_t x_off[G::kXLoads], w_off[2];
  bool x_ok[G::kXLoads];
  int c = 2;  // this wave's copies per stage
#pragma unroll
  for (int i = 0; i < G::kXLoads; ++i) {
    const int t = dma_row(wave, lane, i);
    x_ok[i] = 8 * (uwave + 8 * i) < m_valid;
    c += x_ok[i];
    x_off[i] = static_cast<uint32_t>(slot_src(t)) * K + dma_chunk(t, lane) * 16;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 16 * (wave + 8 * i) + lane / 4;
    const int ch = (lane % 4) ^ ((t >> 2) & 3);
    w_off[i] = static_cast<uint32_t>(wrow_of(t)) * (K / 2) + ch * 16;
  }
  // PER: wave kXsWaves alone copies the weight scale bytes, 16 bytes of 64
  // rows per stage
  const bool s_x = uwave < G::kXsWaves, s_any = uwave < G::kXsWaves + (PER ? 1 : 4);
  c += s_any;
  // activation words: slot t's word of stage kb at xs + 4 (kb n_slots + t),
  // so a stage's rows are one run; weight words: 4 bytes per stage of a row
  auto slot_of = [&](int t) { return min(row0 + t, row_end - 1); };
  const uint8_t* s_src = s_x ? xs + static_cast<int64_t>(slot_of(64 * wave + lane)) * 4
                             : wsb + static_cast<int64_t>(wrow_of(64 * ((s_any ? wave : G::kXsWaves) - G::kXsWaves) + lane)) * (K / 32);
  const int s_step = s_x ? 4 * n_slots : 4;
  const int s_dst = G::kXBytes + G::kWBytes +
                    (s_x ? 256 * wave : BMS * 4 + 256 * ((s_any ? wave : G::kXsWaves) - G::kXsWaves));
  // extension slots: waves 0..3 copy one 8-row region each, wave 0 their
  // scale words (lanes 0-31; the others repeat slot 31 into spare words)
  const int xr = 8 * uwave + lane / 8;
  const bool xt_ok = uwave < 4 && 8 * uwave < x_rows;
  const bool xs_ok = uwave == 0 && x_rows > 0;
  c += xt_ok + xs_ok;
  const uint32_t xt_off = static_cast<uint32_t>(slot_src(BMS + xr)) * K + dma_chunk(xr, lane) * 16;
  const uint8_t* xs_src = xs + static_cast<int64_t>(slot_of(BMS + min(lane, kXtRows - 1))) * 4;
  // PER: with stage kb travel the bytes of period q = kb/kPer + 1 (stages
  // kPer*q ..) of rows 64 g + lane, g = kb % kPer, into buffer q % kPerSlots.
  // That buffer last held period q - 3, read up to stage kPer*(q-2) - 1,
  // before the step that issues stage kb (kb - P >= kPer*(q-2), P <= kPer);
  // periods past the last copy its bytes again into a free buffer.
  const int nper = nk / kPer;
  auto per_src = [&](int g, int q) {
    return wsb + (static_cast<uint32_t>(wrow_of(64 * g + lane)) * (K / 32) + 16 * min(q, nper - 1));
  };
  auto per_dst = [&](int g, int q) { return &lds[kPerOff + (q % kPerSlots) * (BN * 16) + g * 1024]; };
  auto dma = [&](int st, int kb) {
    unsigned char* sb = &lds[st * G::kStage];
#pragma unroll
    for (int i = 0; i < G::kXLoads; ++i)
      if (x_ok[i]) dma16(xq + (x_off[i] + kb * 128), sb + dma_row(wave, 0, i) * 128);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(wb + (w_off[i] + kb * 64), sb + G::kXBytes + (wave + 8 * i) * 1024);
    if (s_any) {
      if (PER && !s_x) dma16(per_src(kb % kPer, kb / kPer + 1), per_dst(kb % kPer, kb / kPer + 1));
      else dma4(s_src + kb * s_step, sb + s_dst);
    }
    if (G::kExt) {
      if (xt_ok) dma16(xq + (xt_off + kb * 128), sb + G::kXtOff + uwave * 1024);
      if (xs_ok) dma4(xs_src + kb * (4 * n_slots), sb + G::kXtOff + kXtRows * 128);
    }
  };
  // scale words of weight row t at stage kb: WS(kb, st)[t * (PER ? 4 : 1)]
  auto ws_of = [&](int kb, int st) {
    return PER ? reinterpret_cast<const uint32_t*>(
                     &lds[kPerOff + ((kb / kPer) % kPerSlots) * (BN * 16)]) + kb % kPer
               : reinterpret_cast<const uint32_t*>(&lds[st * G::kStage + G::kXBytes + G::kWBytes]) + BMS;
  };
  // fragment rows: weights (A) and slots (B)
  int wrow[2], srow[G::kJ];
#pragma unroll
  for (int f = 0; f < 2; ++f)
    wrow[f] = (MODE == kGateUp) ? (f * 128 + wn * 32 + r) : (wn * 64 + f * 32 + r);
#pragma unroll
  for (int j = 0; j < G::kJ; ++j) srow[j] = wm * (BMS / 2) + j * 32 + r;
  f32x16 acc[2][G::kJ];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < G::kJ; ++j) acc[f][j] = f32x16{};
  f32x16 accx = f32x16{};
  // every fragment is full whenever there are extension slots
  const int nj = min(G::kJ, max(0, (m_valid - wm * (BMS / 2) + 31) / 32));
  // the ring, with the fragment count (and whether extension slots take
  // part) fixed per instantiation
  auto run = [&](auto nj_c, auto xt_c) {
    constexpr int NJ = decltype(nj_c)::value;
    constexpr bool XT = decltype(xt_c)::value;
    // period 0 of the weight scale bytes, ahead of stage 0's copies
    if (PER && s_any && !s_x) {
#pragma unroll
      for (int g = 0; g < kPer; ++g) dma16(per_src(g, 0), per_dst(g, 0));
    }
#pragma unroll
    for (int s0 = 0; s0 < P; ++s0)
      if (s0 < nk) dma(s0, s0);
    ring_barrier(c * (min(P, nk) - 1));  // stage 0 landed
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt+P goes to the buffer last read in step kt-1 (ended by a barrier)
      const int kn = kt + P;
      if (kn < nk) dma(st == 0 ? S - 1 : st - 1, kn);
      if (NJ > 0)
        stage_products<BMS, NJ, XT, PER>(&lds[st * G::kStage], ws_of(kt, st), acc, accx, wrow,
                                         srow, half, wm);
      ring_barrier(c * max(0, min(kn, nk - 1) - (kt + 1)));  // stage kt+1 landed
      st = (st == S - 1) ? 0 : st + 1;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, (G::kJ >= 2 ? 2 : 1)>;
  using IJ = std::integral_constant<int, G::kJ>;
  using I3 = std::integral_constant<int, (G::kJ >= 3 ? 3 : (G::kJ >= 2 ? 2 : 1))>;
  using NoX = std::integral_constant<bool, false>;
  using ExtX = std::integral_constant<bool, G::kExt>;
  if (nj == G::kJ && x_rows > 0) run(IJ{}, ExtX{});
  else if (nj == G::kJ) run(IJ{}, NoX{});
  else if (nj == 3) run(I3{}, NoX{});
  else if (nj == 2) run(I2{}, NoX{});
  else if (nj == 1) run(I1{}, NoX{});
  else run(I0{}, NoX{});
  // element q of acc[f][j]: channel row 8*(q/4) + 4*half + q%4 of fragment f,
  // slot row0 + wm*BMS/2 + 32 j + r; elements 4g .. 4g+3 are 4 consecutive
  // channels of the lane's slot.  A gate/up wave's 32 channels are one MXFP8
  // block of h, split over lanes r and r + 32: h is quantised here (fp32
  // value, block exponent from the amax over both lanes) and only its codes
  // and E8M0 byte are written.
#pragma unroll
  for (int j = 0; j < G::kJ; ++j) {
    if (j >= nj) continue;
    const int slot = row0 + wm * (BMS / 2) + j * 32 + r;
    if (MODE == kGateUp) {
      float hv[16];
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        hv[q] = silu(acc[0][j][q]) * acc[1][j][q];
        m = fmaxf(m, fabsf(hv[q]));
      }
      m = fmaxf(m, __shfl_xor(m, 32));
      const int x = mx8_exponent(m);
      if (slot >= row_end) continue;
      uint8_t* hq = static_cast<uint8_t*>(out) + static_cast<int64_t>(slot) * I + nt * 128 + wn * 32;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint32_t*>(hq + 8 * g + 4 * half) =
            e4m3x4(ldexpf(hv[4 * g], -x), ldexpf(hv[4 * g + 1], -x), ldexpf(hv[4 * g + 2], -x),
                   ldexpf(hv[4 * g + 3], -x));
      if (half == 0) out_scale[(static_cast<int64_t>(nt) * n_slots + slot) * 4 + wn] = static_cast<uint8_t>(x + 127);
    } else {
      if (slot >= row_end) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cr = 8 * g + 4 * half;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = nt * BN + wn * 64 + f * 32 + cr;  // H % 128 == 0: all 4 or none
          if (col < H) {
            const f32x4 v = {acc[f][j][4 * g], acc[f][j][4 * g + 1], acc[f][j][4 * g + 2],
                             acc[f][j][4 * g + 3]};
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + static_cast<int64_t>(slot) * H + col) = v;
          }
        }
      }
    }
  }
  if (!G::kExt || x_rows == 0) return;
  // extension slots: accx holds, for slot row0 + BMS + r, channel rows
  // 8*(q/4) + 4*half + q%4 of the wave's fragment wm
  const int slot = row0 + BMS + r;
  if (MODE == kGateUp) {
    // up values (wm = 1) reach the gate waves (wm = 0) of the same channels
    // through LDS, at the same (wn, lane, q) position
    float* ex = reinterpret_cast<float*>(&lds[0]);
    __syncthreads();  // every wave is past its last read of the stages
    if (wm == 1) {
#pragma unroll
      for (int q = 0; q < 16; ++q) ex[(wn * 64 + lane) * 16 + q] = accx[q];
    }
    __syncthreads();
    if (wm == 0) {
      float hv[16];
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        hv[q] = silu(accx[q]) * ex[(wn * 64 + lane) * 16 + q];
        m = fmaxf(m, fabsf(hv[q]));
      }
      m = fmaxf(m, __shfl_xor(m, 32));
      const int x = mx8_exponent(m);
      if (r < x_rows) {
        uint8_t* hq = static_cast<uint8_t*>(out) + static_cast<int64_t>(slot) * I + nt * 128 + wn * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint32_t*>(hq + 8 * g + 4 * half) =
              e4m3x4(ldexpf(hv[4 * g], -x), ldexpf(hv[4 * g + 1], -x), ldexpf(hv[4 * g + 2], -x),
                     ldexpf(hv[4 * g + 3], -x));
        if (half == 0) out_scale[(static_cast<int64_t>(nt) * n_slots + slot) * 4 + wn] = static_cast<uint8_t>(x + 127);
      }
    }
  } else if (r < x_rows) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = nt * BN + wn * 64 + wm * 32 + 8 * g + 4 * half;
      if (col < H) {
        const f32x4 v = {accx[4 * g], accx[4 * g + 1], accx[4 * g + 2], accx[4 * g + 3]};
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + static_cast<int64_t>(slot) * H + col) = v;
      }
    }
  }
}

}  // namespace mxg

// ---- 64-slot tiles with 256-deep stages ---------------------------------------
// For decode batches the 4-bit weights stream from HBM, and a 128-deep stage
// reads each weight row as a 64-byte half of a cache line.  This form takes
// 256 k per stage, so a weight row is one whole 128-byte line per stage (the
// bf16 tiles' row layout, swizzle and copy pattern), with 64 slots x 256
// bytes of activations, in a ring of three 48.5 KiB stages (two in flight)
// with the counted waits of the other rings.  Scale bytes: the activations'
// two words per slot per stage from the block-major slot words (waves 0-1);
// the weights' in periods of two stages, 16 bytes of a row, half of the
// rows with each stage (waves 2-3), in a ring of three 4 KiB buffers after
// the stages (rewritten only after the period it held three periods
// earlier has been read: period q is issued with stages 2(q-1) .. 2q-1 at
// steps >= 2q-4, period q-3 was last read at step 2q-5).  The products
// per 64-deep step are those of the 128-deep form (same operands, same
// order): bit-identical.  K % 512 == 0.
namespace mxw {

using namespace tile;
using mxg::kGateUp;

constexpr int BMS = 64;
constexpr int kXRow = 256;                     // activation bytes per slot per stage
constexpr int kXBytes = BMS * kXRow;           // 16 KiB
constexpr int kWBytes = BN * 128;              // 32 KiB: 256 rows x 128 bytes
constexpr int kXsOff = kXBytes + kWBytes;      // activation scale words [2][64]
constexpr int kStage = kXsOff + 2 * BMS * 4;   // 49,664 bytes
constexpr int kStages = 3, P = kStages - 1;
constexpr int kPerOff = kStages * kStage;
constexpr int kPerSlots = 3;
constexpr int kLds = kPerOff + kPerSlots * BN * 16;  // 161,280 bytes

// 256-byte activation rows: chunk c of slot row t at t * 256 + ((c ^ (t % 16))
// << 4), so 16 consecutive rows at one logical chunk hit distinct banks.
__device__ __forceinline__ int xswz(int t, int c) { return t * kXRow + ((c ^ (t & 15)) << 4); }

template <int MODE>
__global__ __launch_bounds__(tile::kThreads) void grouped_gemm_mx_wide(
    // arguments as for mxg::grouped_gemm_mx
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, void* __restrict__ out,
    uint8_t* __restrict__ out_scale, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ meta, int E, int H, int I,
    int n_nt, int n_slots) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc, BMS, 8, 4)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int nk = K / 256, nper = nk / 2;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int wm = wave / 4, wn = wave % 4, r = lane % 32, half = lane / 32;
  const int m_valid = min(BMS, row_end - row0);
  const int64_t nrows = (MODE == kGateUp) ? 2 * I : H;
  const uint8_t* wb = w + static_cast<int64_t>(e) * nrows * (K / 2);
  const uint8_t* wsb = ws + static_cast<int64_t>(e) * nrows * (K / 32);
  auto wrow_of = [&](int t) {  // weight row of tile row t
    return (MODE == kGateUp) ? ((t < 128) ? nt * 128 + t : I + nt * 128 + (t - 128))
                             : min(nt * BN + t, H - 1);
  };
  auto slot_of = [&](int t) { return min(row0 + t, row_end - 1); };  // padding: a valid slot
  // activations: two 1 KiB regions of 4 rows per wave (lane l writes physical
  // chunk l % 16 of row 4 region + l / 16), copied when the region's first
  // row is valid; weights: four regions of 8 rows (tile::dma_row / dma_chunk)
  uint32_t x_off[2], w_off[4];
  bool x_ok[2];
  int c = 4;  // this wave's copies per stage
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 4 * (wave + 8 * i) + lane / 16;
    x_ok[i] = 4 * (uwave + 8 * i) < m_valid;
    c += x_ok[i];
    const int src = (MODE == kGateUp) ? slot_token[slot_of(t)] : slot_of(t);
    x_off[i] = static_cast<uint32_t>(src) * K + (((lane % 16) ^ (t & 15)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = dma_row(wave, lane, i);
    w_off[i] = static_cast<uint32_t>(wrow_of(t)) * (K / 2) + dma_chunk(t, lane) * 16;
  }
  // scale copies: wave 0 / 1 the slots' word 2 kb / 2 kb + 1 of stage kb;
  // waves 2-3 the weight bytes of period kb/2 + 1 for rows 128 (kb % 2) +
  // 64 (wave - 2) + lane
  const bool s_x = uwave < 2, s_w = uwave == 2 || uwave == 3;
  c += s_x || s_w;
  const uint8_t* xs_src = xs + (static_cast<int64_t>(s_x ? wave : 0) * n_slots + slot_of(lane)) * 4;
  const int wq = s_w ? wave - 2 : 0;
  auto per_src = [&](int g, int q) {
    return wsb + (static_cast<int64_t>(wrow_of(128 * g + 64 * wq + lane)) * (K / 32) +
                  16 * min(q, nper - 1));
  };
  auto per_dst = [&](int g, int q) {
    return &lds[kPerOff + (q % kPerSlots) * (BN * 16) + (128 * g + 64 * wq) * 16];
  };
  auto dma = [&](int st, int kb) {
    unsigned char* sb = &lds[st * kStage];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (x_ok[i]) dma16(xq + (x_off[i] + kb * 256), sb + (wave + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(wb + (w_off[i] + kb * 128), sb + kXBytes + (wave + 8 * i) * 1024);
    if (s_x) dma4(xs_src + static_cast<int64_t>(kb) * (8 * n_slots), sb + kXsOff + wave * 256);
    if (s_w) dma16(per_src(kb % 2, kb / 2 + 1), per_dst(kb % 2, kb / 2 + 1));
  };
  int wrow[2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
    wrow[f] = (MODE == kGateUp) ? (f * 128 + wn * 32 + r) : (wn * 64 + f * 32 + r);
  const int srow = wm * 32 + r;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const bool live = m_valid > wm * 32;  // the wave's 32 slots hold a valid one
  // period 0 of the weight scale bytes, ahead of stage 0's copies
  if (s_w) {
    dma16(per_src(0, 0), per_dst(0, 0));
    dma16(per_src(1, 0), per_dst(1, 0));
  }
#pragma unroll
  for (int s0 = 0; s0 < P; ++s0)
    if (s0 < nk) dma(s0, s0);
  ring_barrier(c * (min(P, nk) - 1));  // stage 0 landed
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int kn = kt + P;
    if (kn < nk) dma(st == 0 ? kStages - 1 : st - 1, kn);
    if (live) {
      const unsigned char* X = &lds[st * kStage];
      const unsigned char* W = X + kXBytes;
      const uint32_t* XS = reinterpret_cast<const uint32_t*>(X + kXsOff);
      const uint32_t* WS = reinterpret_cast<const uint32_t*>(
          &lds[kPerOff + ((kt / 2) % kPerSlots) * (BN * 16)]) + 2 * (kt % 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // scale byte 2 ks + half of the stage: word ks / 2, byte 2 (ks % 2) + half
        const int sh = 8 * (2 * (ks % 2) + half);
        u32x4 a[2];
        uint32_t sa[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          a[f] = *reinterpret_cast<const u32x4*>(W + swz(wrow[f], 2 * ks + half));
          sa[f] = (WS[wrow[f] * 4 + ks / 2] >> sh) & 0xFFu;
        }
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(X + xswz(srow, 4 * ks + half));
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(X + xswz(srow, 4 * ks + 2 + half));
        const uint32_t sb = (XS[(ks / 2) * BMS + srow] >> sh) & 0xFFu;
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[f] = mfma_mx(a[f], b0, b1, acc[f], sa[f], sb);
      }
    }
    ring_barrier(c * max(0, min(kn, nk - 1) - (kt + 1)));  // stage kt+1 landed
    st = (st == kStages - 1) ? 0 : st + 1;
  }
  if (!live) return;
  // epilogue as in mxg::grouped_gemm_mx (one 32-slot fragment per wave)
  const int slot = row0 + srow;
  if (MODE == kGateUp) {
    float hv[16];
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      hv[q] = silu(acc[0][q]) * acc[1][q];
      m = fmaxf(m, fabsf(hv[q]));
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    const int x = mx8_exponent(m);
    if (slot >= row_end) return;
    uint8_t* hq = static_cast<uint8_t*>(out) + static_cast<int64_t>(slot) * I + nt * 128 + wn * 32;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint32_t*>(hq + 8 * g + 4 * half) =
          e4m3x4(ldexpf(hv[4 * g], -x), ldexpf(hv[4 * g + 1], -x), ldexpf(hv[4 * g + 2], -x),
                 ldexpf(hv[4 * g + 3], -x));
    if (half == 0)
      out_scale[(static_cast<int64_t>(nt) * n_slots + slot) * 4 + wn] = static_cast<uint8_t>(x + 127);
  } else {
    if (slot >= row_end) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int cr = 8 * g + 4 * half;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int col = nt * BN + wn * 64 + f * 32 + cr;  // H % 128 == 0: all 4 or none
        if (col < H) {
          const f32x4 v = {acc[f][4 * g], acc[f][4 * g + 1], acc[f][4 * g + 2], acc[f][4 * g + 3]};
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + static_cast<int64_t>(slot) * H + col) = v;
        }
      }
    }
  }
}

}  // namespace mxw

}  // namespace

hipError_t launch_quant_mxfp8(int64_t rows, int64_t cols, int32_t dtype, const void* v,
                              uint8_t* q, uint8_t* scales, hipStream_t s, Timer* tm) {
  const dim3 grid(static_cast<unsigned>(ceil_div(rows * (cols / 32), 256)));
  if (dtype == BEAM_BF16)
    BEAM_LAUNCH(tm, "quant_mxfp8", quant_mxfp8_rows<true>, grid, dim3(256), 0, s, v, rows, cols, q,
                scales, nullptr, 0, nullptr, 0);
  else
    BEAM_LAUNCH(tm, "quant_mxfp8", quant_mxfp8_rows<false>, grid, dim3(256), 0, s, v, rows, cols, q,
                scales, nullptr, 0, nullptr, 0);
  return hipGetLastError();
}

// x -> MXFP8; gate/up with SwiGLU -> h (fp32); h -> MXFP8; down -> y (fp32).
// The grouped gate/up GEMM quantises h in its epilogue; the streaming one
// writes fp32 h for the separate quantiser.
hipError_t launch_experts_mxfp4(const Plan& p, const void* x, const uint8_t* w_gate_up,
                                const uint8_t* s_gate_up, const uint8_t* w_down,
                                const uint8_t* s_down, void* ws, hipStream_t s, Timer* tm) {
  uint8_t* xq = ws_at<uint8_t>(ws, p.off_xq);
  uint8_t* xs = ws_at<uint8_t>(ws, p.off_xs);
  uint8_t* hq = ws_at<uint8_t>(ws, p.off_hq);
  uint8_t* hs = ws_at<uint8_t>(ws, p.off_hs);
  float* h = ws_at<float>(ws, p.off_h);
  float* y = ws_at<float>(ws, p.off_y);
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* active = ws_at<int32_t>(ws, p.off_active);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  const int64_t max_active = p.S < p.E ? p.S : p.E;
  if (!p.stream_path) {
    const int32_t* toff = ws_at<int32_t>(ws, p.off_tile_off);
    const int nt_gu = p.I / 128;
    const int nt_dn = static_cast<int>(ceil_div(p.H, tile::BN));
    uint8_t* xss = ws_at<uint8_t>(ws, p.off_xss);
    const int n_slots = static_cast<int>(p.S);
    // x's E8M0 words also go to its slots, block-major (xss[kb * S + slot])
    BEAM_LAUNCH(tm, "quant_mxfp8", quant_mxfp8_rows<true>,
                dim3(static_cast<unsigned>(ceil_div(p.T * (p.H / 32), 256))), dim3(256), 0, s, x,
                p.T, p.H, xq, xs, ws_at<int32_t>(ws, p.off_slot_of), p.K, xss, n_slots);
#define BEAM_MX_GATE_UP(BMS, STAGES, PER)                                                     \
  BEAM_LAUNCH(tm, "grouped_gate_up_mx", (mxg::grouped_gemm_mx<BMS, STAGES, mxg::kGateUp, PER>), \
              tile::grid_for(p, nt_gu), dim3(tile::kThreads), 0, s, xq, xss, w_gate_up,        \
              s_gate_up, hq, hs, slot_token, counts, offsets, toff, meta, p.E, p.H, p.I, nt_gu, \
              p.xt, n_slots)
#define BEAM_MX_DOWN(BMS, STAGES, PER)                                                        \
  BEAM_LAUNCH(tm, "grouped_down_mx", (mxg::grouped_gemm_mx<BMS, STAGES, mxg::kDown, PER>),     \
              tile::grid_for(p, nt_dn), dim3(tile::kThreads), 0, s, hq, hs, w_down, s_down, y, \
              nullptr, slot_token, counts, offsets, toff, meta, p.E, p.H, p.I, nt_dn, p.xt,    \
              n_slots)
    // weight scale bytes in periods of four stages when K % 512 == 0
#define BEAM_MX_TILES(BMS, STAGES)                                                            \
  if (p.H % 512 == 0) BEAM_MX_GATE_UP(BMS, STAGES, true);                                      \
  else BEAM_MX_GATE_UP(BMS, STAGES, false);                                                    \
  if (p.I % 512 == 0) BEAM_MX_DOWN(BMS, STAGES, true);                                         \
  else BEAM_MX_DOWN(BMS, STAGES, false)
    // measured on the Beam layer: 128-slot tiles (four stages) ahead below
    // 1K tokens; 256-slot tiles with three stages ahead at 1K-4K tokens
    // (2.38 vs 2.46 ms at 4K), with two at 8K (4.24 vs 4.36 ms)
    if (p.bm == 64) {
      // 64-slot tiles: 256-deep stages when K % 512 == 0, else 128-deep
      // stages in a ring of five
      if (p.H % 512 == 0)
        BEAM_LAUNCH(tm, "grouped_gate_up_mx", mxw::grouped_gemm_mx_wide<mxg::kGateUp>,
                    tile::grid_for(p, nt_gu), dim3(tile::kThreads), 0, s, xq, xss, w_gate_up,
                    s_gate_up, hq, hs, slot_token, counts, offsets, toff, meta, p.E, p.H, p.I,
                    nt_gu, n_slots);
      else
        BEAM_MX_GATE_UP(64, 5, false);
      if (p.I % 512 == 0)
        BEAM_LAUNCH(tm, "grouped_down_mx", mxw::grouped_gemm_mx_wide<mxg::kDown>,
                    tile::grid_for(p, nt_dn), dim3(tile::kThreads), 0, s, hq, hs, w_down, s_down,
                    y, nullptr, slot_token, counts, offsets, toff, meta, p.E, p.H, p.I, nt_dn,
                    n_slots);
      else
        BEAM_MX_DOWN(64, 5, false);
    } else if (p.bm == 128) {
      BEAM_MX_TILES(128, 4);
    } else if (p.S < 192 * static_cast<int64_t>(p.E)) {
      BEAM_MX_TILES(256, 3);
    } else {
      BEAM_MX_TILES(256, 2);
    }
#undef BEAM_MX_TILES
#undef BEAM_MX_GATE_UP
#undef BEAM_MX_DOWN
    return hipGetLastError();
  }
  hipError_t e = launch_quant_mxfp8(p.T, p.H, BEAM_BF16, x, xq, xs, s, tm);
  if (e != hipSuccess) return e;
  BEAM_LAUNCH(tm, "stream_gate_up_mx", stream_gate_up_mx,
              dim3(static_cast<unsigned>(ceil_div(max_active * (p.I / 16), kWaves))),
              dim3(kThreads), 0, s, xq, xs, w_gate_up, s_gate_up, h, slot_token, counts,
              offsets, active, meta, p.H, p.I);
  e = launch_quant_mxfp8(p.S, p.I, BEAM_F32, h, hq, hs, s, tm);
  if (e != hipSuccess) return e;
  BEAM_LAUNCH(tm, "stream_down_mx", stream_down_mx,
              dim3(static_cast<unsigned>(ceil_div(max_active * (p.H / 32), kWaves))),
              dim3(kThreads), 0, s, hq, hs, w_down, s_down, y, counts, offsets, active, meta,
              p.H, p.I);
  return hipGetLastError();
}

}  // namespace beam
