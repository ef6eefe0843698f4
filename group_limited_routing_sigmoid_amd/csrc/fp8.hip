// FP8 (OCP e4m3fn) variant of the expert path.  The pages name FP8
// checkpoints ("Hugging Face releases Beam ..." checkpoint paragraph;
// "Reflection Beam", section "Where to run it") without a recipe; this
// library reads it as e4m3fn weights with one fp32 scale per 128x128 block,
// activations quantised per token per 128 channels with scale = amax/448,
// and fp32 accumulation with the scales applied per 128-deep slice.
#include "grouped_tile.h"

namespace beam {
namespace {

// The recipe's block scale: amax / 448 in binary32, or 1 where that is zero
// (an all-zero block, or a subnormal amax whose quotient underflows).
__device__ __forceinline__ float e4m3_scale(float amax) {
  const float sc = amax / 448.0f;
  return sc > 0.0f ? sc : 1.0f;
}

// 16 lanes per (row, 128-column block), 8 consecutive columns per lane (one
// 16-byte load of bf16, two of fp32); a wave covers 4 blocks.  The block's
// amax is reduced over its 16 lanes; scale = e4m3_scale(amax), code =
// e4m3(v / scale) with binary32 division, saturating, as in the recipe.  With
// slot_of (x in the forward) each scale also goes to the K slots of its row,
// block-major: xss[kb * S + slot], so that a tile stage of the grouped
// products reads the scale words of consecutive slots (one 1 KiB run per
// 256 rows rather than a cache line per row).
template <bool BF16>
__global__ __launch_bounds__(256) void quant_e4m3_rows(
    const void* __restrict__ v, int64_t rows, int64_t cols,
    uint8_t* __restrict__ q, float* __restrict__ scales,
    const int32_t* __restrict__ slot_of, int K, float* __restrict__ xss, int S) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8-column group
  const int64_t nbc = cols / 128;
  const int64_t blk = g / 16;
  const bool live = blk < rows * nbc;
  const int64_t at = live ? (blk / nbc) * cols + (blk % nbc) * 128 + (g % 16) * 8 : 0;
  float a[8];
  if (BF16) {
    const u32x4 w = live ? ld16(static_cast<const uint16_t*>(v) + at) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[2 * j] = __uint_as_float(w[j] << 16);
      a[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float* p = static_cast<const float*>(v) + at;
    const u32x4 w0 = live ? ld16(p) : u32x4{0, 0, 0, 0};
    const u32x4 w1 = live ? ld16(p + 4) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = __uint_as_float(w0[j]);
      a[4 + j] = __uint_as_float(w1[j]);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(a[j]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));  // within 16 lanes
  const float sc = e4m3_scale(m);
  const uint32_t lo = e4m3x4(a[0] / sc, a[1] / sc, a[2] / sc, a[3] / sc);
  const uint32_t hi = e4m3x4(a[4] / sc, a[5] / sc, a[6] / sc, a[7] / sc);
  if (!live) return;
  *reinterpret_cast<uint2*>(q + at) = make_uint2(lo, hi);
  if (g % 16 == 0) {
    scales[blk] = sc;
    if (xss) {
      const int64_t row = blk / nbc, kb = blk % nbc;
      for (int k = 0; k < K; ++k) xss[kb * S + slot_of[row * K + k]] = sc;
    }
  }
}

}  // namespace

hipError_t launch_quant_e4m3(int64_t rows, int64_t cols, int32_t dtype,
                             const void* v, uint8_t* q, float* scales,
                             hipStream_t s, Timer* tm) {
  const int64_t groups = rows * (cols / 128) * 16;
  const dim3 grid(static_cast<unsigned>(ceil_div(groups, 256)));
  if (dtype == BEAM_BF16)
    BEAM_LAUNCH(tm, "quant_e4m3", quant_e4m3_rows<true>, grid, dim3(256), 0, s, v, rows, cols, q,
                scales, nullptr, 0, nullptr, 0);
  else
    BEAM_LAUNCH(tm, "quant_e4m3", quant_e4m3_rows<false>, grid, dim3(256), 0, s, v, rows, cols, q,
                scales, nullptr, 0, nullptr, 0);
  return hipGetLastError();
}

bool fp8_experts_built() { return true; }

namespace {

using namespace tile;

enum Mode { kGateUp = 0, kDown = 1 };

// An expert's last M tile may hold 32 extension rows past the 256 (tile rows
// 256..287): their A rows get a 4 KiB tile of their own after the A and B
// tiles of each stage.
constexpr int kXRows = 32;
constexpr int BMX = BM + kXRows;
typedef unsigned char TileLdsX[2][2 * kTileBytes + kXRows * kRowBytes];

// D = A(32x64) * B(64x32) + C on e4m3 codes (format 0, unit E8M0 scales).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, codes
// 32*(l/32) .. +32 of the 64-deep slice; C as for the bf16 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS addresses of the lane's MFMA fragments.  A fragment row is
// base + 32 f (f = fragment index), and with the tile swizzle the physical
// chunk of logical chunk c = 4 hlf + 2 (lane/32) + j of that row is
// ((2 (lane/32) + j) ^ key) ^ 4 ((hlf + f) & 1), key = (l ^ (l >> 3)) & 7 for
// l = lane % 32 (base is a multiple of 64).  So every fragment address is a
// per-lane row offset, one of four per-lane chunk offsets and a constant.
struct FragAddr {
  uint32_t a_row, b_row;  // byte offsets of the lane's A row (f = 0) and B row (n = 0)
  uint32_t x_row;         // byte offset of its row in the extension rows' tile
  uint32_t p[2][2];       // p[j][flip]: chunk byte offset
  uint32_t r_row;         // byte offset of the lane's first ratio (per-row factor)
  uint32_t r_row_x;       // the same for the extension rows (tile rows 256..)
};

// wrows: A rows per wave along M (128, or 64 in the 128-row tiles).
__device__ __forceinline__ FragAddr frag_addr(int wm, int wn, int lane, int wrows = 128) {
  FragAddr fa;
  const int l = lane % 32;
  const int key = (l ^ (l >> 3)) & 7;
  fa.a_row = static_cast<uint32_t>(wm * wrows + l) * kRowBytes;
  fa.b_row = static_cast<uint32_t>(wn * 64 + l) * kRowBytes;
  fa.x_row = static_cast<uint32_t>(l) * kRowBytes;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int f = 0; f < 2; ++f)
      fa.p[j][f] = static_cast<uint32_t>((((2 * (lane / 32) + j) ^ key) ^ (4 * f)) << 4);
  fa.r_row = static_cast<uint32_t>(wm * wrows + 4 * (lane / 32)) * 4;
  fa.r_row_x = static_cast<uint32_t>(BM + 4 * (lane / 32)) * 4;
  return fa;
}

// The lane's 32 codes of 64-deep half hlf of fragment f (32 rows apart).
__device__ __forceinline__ i32x8 frag8(const unsigned char* t, uint32_t row, const FragAddr& fa,
                                       int f, int hlf) {
  const int flip = (hlf + f) & 1;
  const unsigned char* r = t + row + f * 32 * kRowBytes;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(r + fa.p[0][flip]);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(r + fa.p[1][flip]);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// acc[i][n] *= v[row of element] for the 16 rows fragment i holds in this
// lane (v: the per-row factors of the wave's weight block, in LDS).
__device__ __forceinline__ void scale_rows(f32x16 (&acc)[4][2], int i, const float* v,
                                           const FragAddr& fa) {
  const unsigned char* base = reinterpret_cast<const unsigned char*>(v) + fa.r_row;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(base + (i * 32 + 8 * q) * 4);
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][n][4 * q + j] *= t[j];
  }
}

// The same for the extension rows' accumulator.
__device__ __forceinline__ void scale_rows_x(f32x16& accx, const float* v, const FragAddr& fa) {
  const unsigned char* base = reinterpret_cast<const unsigned char*>(v) + fa.r_row_x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(base + 8 * q * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) accx[4 * q + j] *= t[j];
  }
}

// Keeps the compiler from moving instructions, LDS reads included, across
// this point (a scheduling fence alone lets it hoist every read of the stage
// to the top, and the registers holding them then spill).
__device__ __forceinline__ void fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Ties the value to this point of the instruction stream (the matrix
// products are pure computations the compiler would otherwise move freely).
__device__ __forceinline__ void pin(f32x16& v) { asm volatile("" : "+v"(v)); }

// t: the factors (per-row rescale ratios) of the 16 rows fragment i holds
// in this lane, four 16-byte reads of the factor table v.
__device__ __forceinline__ void read_factors(f32x4 (&t)[4], int i, const float* v,
                                             const FragAddr& fa) {
  const unsigned char* base = reinterpret_cast<const unsigned char*>(v) + fa.r_row;
#pragma unroll
  for (int q = 0; q < 4; ++q) t[q] = *reinterpret_cast<const f32x4*>(base + (i * 32 + 8 * q) * 4);
}
// a *= t[row of element] for one 32x32 accumulator of that fragment.
__device__ __forceinline__ void mul_factors(f32x16& a, const f32x4 (&t)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) a[4 * q + j] *= t[q][j];
}

// One 128-deep stage for the wave's first NF fragments: add the stage's
// exact products, one 64-deep half at a time (B fragments of the half held,
// A fragments read one ahead), then rescale the accumulators to the next
// stage's scale (factors `next`, 1 after the last stage).  The rescale of
// fragment i goes between the products of fragment i+1 (one multiply
// group beside each product), so the multiplies overlap the matrix-core
// work instead of holding up the products that need them; each sum still
// sees the same operations in the same order (products of stage kb, then
// the factor of kb+1, then products of kb+1).
// XT: the tile also holds extension rows (tile rows 256..287, their own
// 4 KiB tile xt); wave (wm, wn) adds their products with its B fragment wm,
// i.e. columns wn*64 + wm*32 .. +32, into accx.
template <int NF, bool XT, typename Copy>
__device__ __forceinline__ void fp8_stage(const unsigned char* at, const unsigned char* bt,
                                          const unsigned char* xt, const float* next,
                                          f32x16 (&acc)[4][2], f32x16& accx, int wm,
                                          const FragAddr& fa, Copy&& copy) {
  {  // first 64-deep half: products, the next stage's weight copies between them
    const i32x8 b0 = frag8(bt, fa.b_row, fa, 0, 0);
    const i32x8 b1 = frag8(bt, fa.b_row, fa, 1, 0);
    if (XT) {
      const i32x8 ax = frag8(xt, fa.x_row, fa, 0, 0);
      accx = mfma_fp8_32x32x64(ax, wm ? b1 : b0, accx);
      pin(accx);
    }
    i32x8 a = frag8(at, fa.a_row, fa, 0, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      i32x8 an = a;
      if (i + 1 < NF) an = frag8(at, fa.a_row, fa, i + 1, 0);
      acc[i][0] = mfma_fp8_32x32x64(a, b0, acc[i][0]);
      pin(acc[i][0]);
      copy(i);
      acc[i][1] = mfma_fp8_32x32x64(a, b1, acc[i][1]);
      pin(acc[i][1]);
      a = an;
    }
#pragma unroll
    for (int c = NF; c < 4; ++c) copy(c);
  }
  fence();
  {  // second half: products, fragment i-1's rescale and the next stage's
     // token-row copies beside fragment i's
    const i32x8 b0 = frag8(bt, fa.b_row, fa, 0, 1);
    const i32x8 b1 = frag8(bt, fa.b_row, fa, 1, 1);
    if (XT) {
      const i32x8 ax = frag8(xt, fa.x_row, fa, 0, 1);
      accx = mfma_fp8_32x32x64(ax, wm ? b1 : b0, accx);
      pin(accx);
    }
    i32x8 a = frag8(at, fa.a_row, fa, 0, 1);
    f32x4 t[4];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      i32x8 an = a;
      if (i + 1 < NF) an = frag8(at, fa.a_row, fa, i + 1, 1);
      acc[i][0] = mfma_fp8_32x32x64(a, b0, acc[i][0]);
      pin(acc[i][0]);
      if (i > 0) {
        mul_factors(acc[i - 1][0], t);
        pin(acc[i - 1][0]);
      }
      acc[i][1] = mfma_fp8_32x32x64(a, b1, acc[i][1]);
      pin(acc[i][1]);
      copy(4 + i);
      if (i > 0) {
        mul_factors(acc[i - 1][1], t);
        pin(acc[i - 1][1]);
      }
      fence();
      read_factors(t, i, next, fa);
      fence();
      a = an;
    }
#pragma unroll
    for (int c = 4 + NF; c < 9; ++c) copy(c);
    if (NF > 0) {
      mul_factors(acc[NF - 1][0], t);
      pin(acc[NF - 1][0]);
      mul_factors(acc[NF - 1][1], t);
      pin(acc[NF - 1][1]);
    }
    if (XT) {
      fence();
      scale_rows_x(accx, next, fa);
      pin(accx);
    }
  }
}

// The 128-row tiles' stage (factors of the stage itself, applied first):
// for the wave's first NF fragments rescale the
// accumulators to this stage's scale and add the stage's exact products, one
// 64-deep half at a time (B fragments of the half held, A fragments read one
// ahead).  Fragment i is rescaled just before its first product of the
// stage, so the multiplies overlap the matrix-core work of fragment i-1.
// XT: the tile also holds extension rows (tile rows 256..287, their own
// 4 KiB tile xt); wave (wm, wn) adds their products with its B fragment wm,
// i.e. columns wn*64 + wm*32 .. +32, into accx.
template <int NF, bool XT>
__device__ __forceinline__ void fp8_stage_pre(const unsigned char* at, const unsigned char* bt,
                                              const unsigned char* xt, const float* ratio,
                                              f32x16 (&acc)[4][2], f32x16& accx, int wm,
                                              const FragAddr& fa) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const i32x8 b0 = frag8(bt, fa.b_row, fa, 0, h);
    const i32x8 b1 = frag8(bt, fa.b_row, fa, 1, h);
    if (XT) {
      const i32x8 ax = frag8(xt, fa.x_row, fa, 0, h);
      if (h == 0) scale_rows_x(accx, ratio, fa);
      accx = mfma_fp8_32x32x64(ax, wm ? b1 : b0, accx);
    }
    i32x8 a = frag8(at, fa.a_row, fa, 0, h);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      i32x8 an = a;
      if (i + 1 < NF) an = frag8(at, fa.a_row, fa, i + 1, h);
      if (h == 0) scale_rows(acc, i, ratio, fa);
      acc[i][0] = mfma_fp8_32x32x64(a, b0, acc[i][0]);
      acc[i][1] = mfma_fp8_32x32x64(a, b1, acc[i][1]);
      a = an;
    }
  }
}

// Main loop over the K/128 stages.  Block scales: the exact product of a
// 128-deep stage kb is P_kb (unit scales); the result is sum_kb s_kb * P_kb
// with s_kb = s_a[row, kb] * s_w[block, kb].  The accumulator is kept in units
// of the current stage's s: between P_{kb-1} and P_kb it is multiplied by
// s_{kb-1} / s_kb (at the end of stage kb-1), and the epilogue multiplies by
// the last s.  Each thread computes the factors of its (weight block, tile
// row) items two stages ahead into rsc[stage % 2]: (tid / 256, tid % 256),
// and, in a tile with extension rows (XT),
// for threads 0..63 also an extension row (tid / 32, 256 + tid % 32) (the
// others repeat their first item).  s_last receives the items' last s.
struct ScaleItems {
  const float* sa[2];  // s_a of the item's slot at block 0; block kb at kb * S
  const float* sw[2];  // s_w of the item's weight block, one word per block
  int blk[2], row[2];
  int S;
};

template <int NF, bool XT>
__device__ __forceinline__ void fp8_mainloop(
    const uint8_t* __restrict__ a_src, const uint32_t* a_off, const bool* a_ok,
    uint32_t x_off, bool x_ok, const uint8_t* __restrict__ wb, const uint32_t* b_off,
    const ScaleItems& it, int nkb, TileLdsX& lds, float (&rsc)[2][2][BMX],
    f32x16 (&acc)[4][2], f32x16& accx, const FragAddr& fa, int wm, int wn, float (&s_last)[2]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto dma = [&](int buf, int kb) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int region = wave + 8 * i;
      if (a_ok[i]) dma16(a_src + (a_off[i] + kb * 128), &lds[buf][region * 1024]);
      dma16(wb + (b_off[i] + kb * 128), &lds[buf][kTileBytes + region * 1024]);
    }
    if (x_ok) dma16(a_src + (x_off + kb * 128), &lds[buf][2 * kTileBytes + wave * 1024]);
  };
  constexpr int NI = XT ? 2 : 1;  // scale items per thread
  dma(0, 0);
  // factors of stage 1 (1 if there is none), applied after stage 0's
  // products; words of stage 2, for the factors of stage 2
  float s_prev[NI], sa_n[NI], sw_n[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const float s0 = it.sa[j][0] * it.sw[j][0];
    const float s1 = it.sa[j][min(1, nkb - 1) * it.S] * it.sw[j][min(1, nkb - 1)];
    rsc[1][it.blk[j]][it.row[j]] = (nkb > 1) ? s0 / s1 : 1.0f;
    s_prev[j] = (nkb > 1) ? s1 : s0;
    sa_n[j] = it.sa[j][min(2, nkb - 1) * it.S];
    sw_n[j] = it.sw[j][min(2, nkb - 1)];
  }
  __syncthreads();
  for (int kt = 0; kt < nkb; ++kt) {
    const int buf = kt & 1;
    // buffer buf^1 was last read before the barrier that ended step kt-1;
    // rsc[buf^1] holds the factors of stage kt+1, rsc[buf] (those of stage
    // kt, read in step kt-1) takes those of stage kt+2 below.
    //
    // Copies of stage kt+1, spread over the stage's products (copies 0-3:
    // the wave's weight regions, one beside every other product of the first
    // half, so the bytes from HBM get the longest lead; 4-7: its token-row
    // regions, which the L2 mostly holds, beside the second half's; 8: the
    // extension rows' region): a compute unit's texture path takes about 64
    // bytes a cycle, and eight waves issuing all their copies at the top of
    // the stage stall at issue (measured at 8K tokens, gate/up: 2.56 ms with
    // the burst, 2.43 with every copy in the first half, 2.37 split so)
    const bool more = kt + 1 < nkb;
    auto copy = [&](int c) {
      if (!more) return;
      unsigned char* nb = &lds[buf ^ 1][0];
      const int kb = kt + 1;
      if (c < kLoads) {
        dma16(wb + (b_off[c] + kb * 128), nb + kTileBytes + (wave + 8 * c) * 1024);
      } else if (c < 2 * kLoads) {
        const int i = c - kLoads;
        if (a_ok[i]) dma16(a_src + (a_off[i] + kb * 128), nb + (wave + 8 * i) * 1024);
      } else if (x_ok) {
        dma16(a_src + (x_off + kb * 128), nb + 2 * kTileBytes + wave * 1024);
      }
    };
    // scale words of stage kt+3 (for the factors of kt+3, formed in step kt+1)
    const int k3 = min(kt + 3, nkb - 1);
    float sa3[NI], sw3[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      sa3[j] = it.sa[j][k3 * it.S];
      sw3[j] = it.sw[j][k3];
    }
    // no branch from here to the barrier, so the compiler keeps the
    // stage's reads next to the products that use them
    if (NF > 0)
      fp8_stage<NF, XT>(&lds[buf][0], &lds[buf][kTileBytes], &lds[buf][2 * kTileBytes],
                        &rsc[buf ^ 1][wn / 2][0], acc, accx, wm, fa, copy);
    else
      for (int c = 0; c < 9; ++c) copy(c);
    // The factor arithmetic waits for its inputs with the wave's whole
    // vector-memory count, stage kt+1's copies included: keep it after the
    // products (the barrier below waits for those copies anyway).
    __builtin_amdgcn_sched_barrier(0);
    // factors of stage kt+2 (1 past the last stage)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const float s = sa_n[j] * sw_n[j];
      const bool real = kt + 2 < nkb;
      rsc[buf][it.blk[j]][it.row[j]] = real ? s_prev[j] / s : 1.0f;
      s_prev[j] = real ? s : s_prev[j];
      sa_n[j] = sa3[j];
      sw_n[j] = sw3[j];
    }
    __syncthreads();  // waits for this wave's loads, then for every wave
  }
  s_last[0] = s_prev[0];
  s_last[1] = s_prev[NI - 1];
}

// Grouped e4m3 GEMM with per-128 block scales.  Same work list, tile
// layout, DMA pattern and XCD order as the bf16 grouped GEMM: 256x256 tiles,
// 128 codes deep per stage, 8 waves of 128x64.  Each wave's 64 columns lie in
// one 128-row block of weight scales: waves 0-1 hold gate channels and 2-3
// the matching up channels of a gate/up tile (128 channels), whose up values
// reach the gate waves through LDS for silu(g)*u.  A gate/up tile holds one
// whole 128-channel block of h for each of its rows, so it also quantises h
// (bf16 value, then the activation recipe) and writes codes and scales.
template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8(
    const uint8_t* __restrict__ a_src,   // gate/up: xq [T,H]; down: hq [S,I]
    const float* __restrict__ a_scale,   // gate/up: xss [H/128,S]; down: hs [I/128,S]
    const uint8_t* __restrict__ w,       // W_gu [E,2I,H] or W_d [E,H,I] codes
    const float* __restrict__ w_scale,   // [E,2I/128,H/128] or [E,H/128,I/128]
    void* __restrict__ out,              // gate/up: hq [S,I] codes; down: y [S,H] bf16
    float* __restrict__ out_scale,       // gate/up: hs [I/128,S]; down: unused
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ meta, int E, int H, int I, int n_nt, int xt, int S) {
  __shared__ __attribute__((aligned(16))) TileLdsX lds;
  __shared__ __attribute__((aligned(16))) float rsc[2][2][BMX];

  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int nkb = K / 128;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 4, wn = wave % 4;
  const int m_valid = min(BM, row_end - row0);
  // extension rows: only in an expert's last tile, when tiles may extend
  // (a tile with more than BM + xt rows left is not the last)
  const int m_all = row_end - row0;
  const int x_rows = (m_all > BM && m_all <= BM + xt) ? m_all - BM : 0;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy

  const uint8_t* wb = w + static_cast<int64_t>(e) * ((MODE == kGateUp) ? 2 * I : H) * K;
  uint32_t a_off[kLoads], b_off[kLoads];
  bool a_ok[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = dma_row(wave, lane, i);
    const int c = dma_chunk(r, lane);
    a_ok[i] = r < m_valid;
    const int slot = min(row0 + r, row_end - 1);  // padded rows: any valid row
    a_off[i] = ((MODE == kGateUp) ? static_cast<uint32_t>(slot_token[slot]) * H
                                  : static_cast<uint32_t>(slot) * I) + c * 16;
    // gate/up: rows 0..127 gate channels nt*128 + r, rows 128..255 the up
    // channels; down: weight row nt*256 + r (the last tile may pass H)
    const int wrow = (MODE == kGateUp) ? ((r < 128) ? nt * 128 + r : I + nt * 128 + (r - 128))
                                       : min(nt * BN + r, H - 1);
    b_off[i] = static_cast<uint32_t>(wrow) * K + c * 16;
  }
  // extension rows' copies: waves 0..3, one 8-row region each
  const int xr = 8 * uwave + lane / 8;
  const bool x_ok = uwave < 4 && 8 * uwave < x_rows;
  const uint32_t x_off =
      ((MODE == kGateUp) ? static_cast<uint32_t>(slot_token[min(row0 + BM + xr, row_end - 1)]) * H
                         : static_cast<uint32_t>(min(row0 + BM + xr, row_end - 1)) * I) +
      dma_chunk(xr, lane) * 16;
  // scale items: (weight block, tile row)
  const int nrb = (MODE == kGateUp) ? 2 * I / 128 : H / 128;
  ScaleItems it;
  it.S = S;
  it.blk[0] = tid / BM;
  it.row[0] = tid % BM;
  it.blk[1] = (tid < 2 * kXRows) ? tid / kXRows : it.blk[0];
  it.row[1] = (tid < 2 * kXRows) ? BM + tid % kXRows : it.row[0];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    it.sa[j] = a_scale + min(row0 + it.row[j], row_end - 1);
    const int wblock = (MODE == kGateUp) ? (it.blk[j] == 0 ? nt : I / 128 + nt)
                                         : min(2 * nt + it.blk[j], nrb - 1);
    it.sw[j] = w_scale + (static_cast<int64_t>(e) * nrb + wblock) * nkb;
  }

  // A rows of this wave: wm*128 + 32 i + lane%32; B rows: wn*64 + 32 n + lane%32
  const FragAddr fa = frag_addr(wm, wn, lane);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};
  f32x16 accx = f32x16{};

  const int nf = wave_frags(m_valid, wm);  // 4 whenever there are extension rows
  float s_last[2];
#define BEAM_FP8_LOOP(NF, XT)                                                                 \
  fp8_mainloop<NF, XT>(a_src, a_off, a_ok, x_off, x_ok, wb, b_off, it, nkb, lds, rsc, acc, \
                       accx, fa, wm, wn, s_last)
  switch (nf) {
    case 4:
      if (x_rows > 0) BEAM_FP8_LOOP(4, true);
      else BEAM_FP8_LOOP(4, false);
      break;
    case 3: BEAM_FP8_LOOP(3, false); break;
    case 2: BEAM_FP8_LOOP(2, false); break;
    case 1: BEAM_FP8_LOOP(1, false); break;
    default: BEAM_FP8_LOOP(0, false); break;
  }
#undef BEAM_FP8_LOOP

  // ---- epilogue: last stage's scale, then store ---------------------------
  // rsc is no longer read by the main loop
  rsc[0][it.blk[0]][it.row[0]] = s_last[0];
  rsc[0][it.blk[1]][it.row[1]] = s_last[1];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nf) scale_rows(acc, i, &rsc[0][wn / 2][0], fa);
  if (x_rows > 0) scale_rows_x(accx, &rsc[0][wn / 2][0], fa);

  if (MODE == kGateUp) {
    // up values, fp32, [256 rows][128 channels] over the two tile buffers
    float* ex = reinterpret_cast<float*>(&lds[0][0]);
    if (wn >= 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nf) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
#pragma unroll
          for (int n = 0; n < 2; ++n)
            ex[rl * 128 + (wn - 2) * 64 + n * 32 + lane % 32] = acc[i][n][r];
        }
      }
    }
    __syncthreads();
    // h = bf16(silu(g) * u), written over the up value it was made from
    if (wn < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nf) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int at = rl * 128 + wn * 64 + n * 32 + lane % 32;
            const float h = silu(acc[i][n][r]) * ex[at];
            ex[at] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(h)) << 16);
          }
        }
      }
    }
    __syncthreads();
    // 16 lanes per row, 8 channels each; amax over the row's 16 lanes
    uint8_t* hq = static_cast<uint8_t*>(out);
#pragma unroll 1
    for (int rl = tid / 16; rl < BM; rl += kThreads / 16) {
      const int c8 = 8 * (tid % 16);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8 + 4]);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(v0[j]), fabsf(v1[j])));
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float sc = e4m3_scale(m);
      const uint32_t lo = e4m3x4(v0[0] / sc, v0[1] / sc, v0[2] / sc, v0[3] / sc);
      const uint32_t hi = e4m3x4(v1[0] / sc, v1[1] / sc, v1[2] / sc, v1[3] / sc);
      if (row0 + rl < row_end) {
        const int64_t row = row0 + rl;
        *reinterpret_cast<uint2*>(hq + row * I + nt * 128 + c8) = make_uint2(lo, hi);
        if (tid % 16 == 0) out_scale[static_cast<int64_t>(nt) * S + row] = sc;
      }
    }
    if (x_rows > 0) {
      // extension rows (32 x 128 channels): wave (wm, wn) holds channels
      // (wn % 2)*64 + wm*32 .. +32, gate for wn < 2 and up for wn >= 2
      __syncthreads();  // every read of ex above is done
      if (wn >= 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
          ex[rl * 128 + (wn - 2) * 64 + wm * 32 + lane % 32] = accx[r];
        }
      }
      __syncthreads();
      if (wn < 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
          const int at = rl * 128 + wn * 64 + wm * 32 + lane % 32;
          const float h = silu(accx[r]) * ex[at];
          ex[at] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(h)) << 16);
        }
      }
      __syncthreads();
      const int rl = tid / 16, c8 = 8 * (tid % 16);  // 32 rows, one pass
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8 + 4]);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(v0[j]), fabsf(v1[j])));
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float sc = e4m3_scale(m);
      const uint32_t lo = e4m3x4(v0[0] / sc, v0[1] / sc, v0[2] / sc, v0[3] / sc);
      const uint32_t hi = e4m3x4(v1[0] / sc, v1[1] / sc, v1[2] / sc, v1[3] / sc);
      if (rl < x_rows) {
        const int64_t row = row0 + BM + rl;
        *reinterpret_cast<uint2*>(hq + row * I + nt * 128 + c8) = make_uint2(lo, hi);
        if (tid % 16 == 0) out_scale[static_cast<int64_t>(nt) * S + row] = sc;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nf) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (row >= row_end) continue;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = nt * BN + wn * 64 + n * 32 + lane % 32;
          if (col < H)
            static_cast<uint16_t*>(out)[static_cast<int64_t>(row) * H + col] =
                f32_to_bf16_bits(acc[i][n][r]);
        }
      }
    }
    if (x_rows > 0) {
      const int col = nt * BN + wn * 64 + wm * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (rl < x_rows && col < H)
          static_cast<uint16_t*>(out)[static_cast<int64_t>(row0 + BM + rl) * H + col] =
              f32_to_bf16_bits(accx[r]);
      }
    }
  }
}

// ---- 128-row tiles with a ring of three copy stages --------------------------
// For batches whose experts hold few rows the e4m3 products are bound by the
// weight bytes.  As in the bf16 128-row form, 128 x 256 tiles are copied
// through a ring of three stages (two in flight while one is consumed),
// each wave issuing the same count of copies per stage so that a stage's
// arrival is a count of outstanding copies.  The per-128 scale words travel
// in the same copies (no global load sits in the loop, whose wait would
// drain the ring): stage kt's buffer also holds s_a of the tile's rows and
// the two s_w words of block kt+1, from which the factors of block kt+1 are
// formed during stage kt.  8 waves of 64 x 64.
namespace small8 {

constexpr int BMS = 128;
constexpr int kABytes = BMS * kRowBytes;             // 16 KiB
constexpr int kSaOff = kABytes + kTileBytes;         // s_a words of the tile's rows
constexpr int kSwOff = kSaOff + BMS * 4;             // s_w words (2 used)
constexpr int kStage = kSwOff + 256;                 // 49,920 bytes
constexpr int kStages = 3;
constexpr int kALoads = kABytes / (16 * kThreads);   // 2
typedef unsigned char Ring[kStages][kStage];

template <int NF>
__device__ __forceinline__ float mainloop(
    const uint8_t* __restrict__ a_src, const uint32_t* a_off, const bool* a_ok, int c,
    const uint8_t* __restrict__ wb, const uint32_t* b_off, const float* sc_src, int sc_stride,
    bool sc_wave, int sc_dst, float s0, int nkb, Ring& ring, float (&rsc)[2][2][BMS], int blk, int srow,
    f32x16 (&acc)[4][2], const FragAddr& fa, int wn) {
  const int wave = threadIdx.x / kWave;
  f32x16 accx = {};
  auto dma = [&](int st, int kb) {
#pragma unroll
    for (int i = 0; i < kALoads; ++i)
      if (a_ok[i]) dma16(a_src + (a_off[i] + kb * 128), &ring[st][(wave + 8 * i) * 1024]);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      dma16(wb + (b_off[i] + kb * 128), &ring[st][kABytes + (wave + 8 * i) * 1024]);
    // scale words of block kb+1 (the last stage repeats block nkb-1)
    if (sc_wave) dma4(sc_src + min(kb + 1, nkb - 1) * sc_stride, &ring[st][sc_dst]);
  };
  rsc[0][blk][srow] = 1.0f;
  float s_prev = s0;
#pragma unroll
  for (int k0 = 0; k0 < 2; ++k0)
    if (k0 < nkb) dma(k0, k0);
  ring_barrier(c * (min(2, nkb) - 1));  // stage 0 landed, rsc[0] written
  int st = 0;
  for (int kt = 0; kt < nkb; ++kt) {
    const int kn = kt + 2;
    if (kn < nkb) dma(st == 0 ? 2 : st - 1, kn);  // the buffer read in step kt-1
    if (NF > 0)
      fp8_stage_pre<NF, false>(&ring[st][0], &ring[st][kABytes], nullptr,
                               &rsc[kt & 1][wn / 2][0], acc, accx, 0, fa);
    __builtin_amdgcn_sched_barrier(0);
    // factors of block kt+1 from this stage's scale words; rsc[(kt+1) & 1]
    // was last read in step kt-1
    const float* sa = reinterpret_cast<const float*>(&ring[st][kSaOff]);
    const float* sw = reinterpret_cast<const float*>(&ring[st][kSwOff]);
    const float s = sa[srow] * sw[blk];
    rsc[(kt + 1) & 1][blk][srow] = s_prev / s;
    s_prev = (kt + 1 < nkb) ? s : s_prev;
    ring_barrier(c * max(0, min(kn, nkb - 1) - (kt + 1)));  // stage kt+1 landed
    st = (st == 2) ? 0 : st + 1;
  }
  return s_prev;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8_small(
    // arguments as for grouped_gemm_fp8: a_scale and out_scale [K/128][S]
    // (S slots), per slot and block-major
    const uint8_t* __restrict__ a_src, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale, void* __restrict__ out,
    float* __restrict__ out_scale, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ meta, int E, int H, int I,
    int n_nt, int S) {
  __shared__ __attribute__((aligned(16))) Ring ring;
  __shared__ __attribute__((aligned(16))) float rsc[2][2][BMS];

  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc, BMS)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int nkb = K / 128;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int wm = wave / 4, wn = wave % 4;
  const int m_valid = min(BMS, row_end - row0);
  const uint8_t* wb = w + static_cast<int64_t>(e) * ((MODE == kGateUp) ? 2 * I : H) * K;
  auto arow_of = [&](int t) {  // activation row of tile row t (padding rows: a valid one)
    const int sl = min(row0 + t, row_end - 1);
    return (MODE == kGateUp) ? slot_token[sl] : sl;
  };
  const int nrb = (MODE == kGateUp) ? 2 * I / 128 : H / 128;
  auto wblock_of = [&](int b) {
    return (MODE == kGateUp) ? (b == 0 ? nt : I / 128 + nt) : min(2 * nt + b, nrb - 1);
  };
  uint32_t a_off[kALoads], b_off[kLoads];
  bool a_ok[kALoads];
  int c = kLoads;  // copies per stage: B regions, valid A regions, scale words
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r = dma_row(wave, lane, i);
    a_ok[i] = 8 * (uwave + 8 * i) < m_valid;  // the region's first row is valid
    c += a_ok[i];
    a_off[i] = static_cast<uint32_t>(arow_of(r)) * K + dma_chunk(r, lane) * 16;
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = dma_row(wave, lane, i);
    const int wrow = (MODE == kGateUp) ? ((r < 128) ? nt * 128 + r : I + nt * 128 + (r - 128))
                                       : min(nt * BN + r, H - 1);
    b_off[i] = static_cast<uint32_t>(wrow) * K + dma_chunk(r, lane) * 16;
  }
  // scale words: waves 0-1 s_a of tile rows 64 w + lane (the slots' words
  // of a block are consecutive: stride S from block to block), wave 2 s_w of
  // the two weight blocks (lanes 0-1; the others repeat block 1 into spare
  // words; one word per block)
  const bool sc_wave = uwave < 3;
  c += sc_wave;
  auto slot_of = [&](int t) { return min(row0 + t, row_end - 1); };
  const float* sc_src = (wave < 2)
      ? a_scale + slot_of(64 * wave + lane)
      : w_scale + (static_cast<int64_t>(e) * nrb + wblock_of(min(lane, 1))) * nkb;
  const int sc_stride = (wave < 2) ? S : 1;
  const int sc_dst = (wave < 2) ? kSaOff + 256 * wave : kSwOff;
  // scale items: threads 0..255 (weight block tid / 128, tile row tid % 128);
  // threads 256.. repeat them
  const int blk = (tid % 256) / BMS, srow = tid % BMS;
  const float s0 = a_scale[slot_of(srow)] *
                   w_scale[(static_cast<int64_t>(e) * nrb + wblock_of(blk)) * nkb];

  const FragAddr fa = frag_addr(wm, wn, lane, 64);
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};
  const int nf = min(2, max(0, (m_valid - wm * 64 + 31) / 32));
  float s_last;
  switch (nf) {
    case 2: s_last = mainloop<2>(a_src, a_off, a_ok, c, wb, b_off, sc_src, sc_stride, sc_wave, sc_dst, s0, nkb, ring, rsc, blk, srow, acc, fa, wn); break;
    case 1: s_last = mainloop<1>(a_src, a_off, a_ok, c, wb, b_off, sc_src, sc_stride, sc_wave, sc_dst, s0, nkb, ring, rsc, blk, srow, acc, fa, wn); break;
    default: s_last = mainloop<0>(a_src, a_off, a_ok, c, wb, b_off, sc_src, sc_stride, sc_wave, sc_dst, s0, nkb, ring, rsc, blk, srow, acc, fa, wn); break;
  }

  // ---- epilogue: last block's scale, then store ---------------------------
  rsc[0][blk][srow] = s_last;  // rsc is no longer read by the main loop
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < nf) scale_rows(acc, i, &rsc[0][wn / 2][0], fa);

  if (MODE == kGateUp) {
    // up values, fp32, [128 rows][128 channels] in the ring buffers
    float* ex = reinterpret_cast<float*>(&ring[0][0]);
    if (wn >= 2) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i >= nf) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
#pragma unroll
          for (int n = 0; n < 2; ++n)
            ex[rl * 128 + (wn - 2) * 64 + n * 32 + lane % 32] = acc[i][n][r];
        }
      }
    }
    __syncthreads();
    // h = bf16(silu(g) * u), written over the up value it was made from
    if (wn < 2) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i >= nf) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int at = rl * 128 + wn * 64 + n * 32 + lane % 32;
            const float h = silu(acc[i][n][r]) * ex[at];
            ex[at] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(h)) << 16);
          }
        }
      }
    }
    __syncthreads();
    // 16 lanes per row, 8 channels each; amax over the row's 16 lanes
    uint8_t* hq = static_cast<uint8_t*>(out);
#pragma unroll 1
    for (int rl = tid / 16; rl < BMS; rl += kThreads / 16) {
      const int c8 = 8 * (tid % 16);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&ex[rl * 128 + c8 + 4]);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(v0[j]), fabsf(v1[j])));
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float sc = e4m3_scale(m);
      const uint32_t lo = e4m3x4(v0[0] / sc, v0[1] / sc, v0[2] / sc, v0[3] / sc);
      const uint32_t hi = e4m3x4(v1[0] / sc, v1[1] / sc, v1[2] / sc, v1[3] / sc);
      if (row0 + rl < row_end) {
        const int64_t row = row0 + rl;
        *reinterpret_cast<uint2*>(hq + row * I + nt * 128 + c8) = make_uint2(lo, hi);
        if (tid % 16 == 0) out_scale[static_cast<int64_t>(nt) * S + row] = sc;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nf) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (row >= row_end) continue;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = nt * BN + wn * 64 + n * 32 + lane % 32;
          if (col < H)
            static_cast<uint16_t*>(out)[static_cast<int64_t>(row) * H + col] =
                f32_to_bf16_bits(acc[i][n][r]);
        }
      }
    }
  }
}

}  // namespace small8

}  // namespace

// x -> e4m3 (per token, per 128 channels); gate/up GEMM with SwiGLU, h
// rounded to bf16 and quantised to e4m3 (per slot, per 128 channels) in its
// epilogue; down GEMM -> y (bf16).
hipError_t launch_experts_fp8(const Plan& p, const void* x,
                              const uint8_t* w_gate_up, const float* s_gate_up,
                              const uint8_t* w_down, const float* s_down,
                              void* ws, hipStream_t s, Timer* tm) {
  uint8_t* xq = ws_at<uint8_t>(ws, p.off_xq);
  float* xs = ws_at<float>(ws, p.off_xs);
  uint8_t* hq = ws_at<uint8_t>(ws, p.off_hq);
  float* hs = ws_at<float>(ws, p.off_hs);
  uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* toff = ws_at<int32_t>(ws, p.off_tile_off);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  float* xss = ws_at<float>(ws, p.off_xss);
  const int32_t* slot_of = ws_at<int32_t>(ws, p.off_slot_of);
  const int S = static_cast<int>(p.S);
  BEAM_LAUNCH(tm, "quant_e4m3", quant_e4m3_rows<true>,
              dim3(static_cast<unsigned>(ceil_div(p.T * (p.H / 128) * 16, 256))), dim3(256), 0, s,
              x, p.T, p.H, xq, xs, slot_of, p.K, xss, S);
  const int nt_gu = p.I / 128;
  const int nt_dn = static_cast<int>(ceil_div(p.H, BN));
  if (p.bm == small8::BMS) {
    BEAM_LAUNCH(tm, "gate_up_fp8", small8::grouped_gemm_fp8_small<kGateUp>, grid_for(p, nt_gu),
                dim3(kThreads), 0, s, xq, xss, w_gate_up, s_gate_up, hq, hs, slot_token, counts,
                offsets, toff, meta, p.E, p.H, p.I, nt_gu, S);
    BEAM_LAUNCH(tm, "down_fp8", small8::grouped_gemm_fp8_small<kDown>, grid_for(p, nt_dn),
                dim3(kThreads), 0, s, hq, hs, w_down, s_down, y, nullptr, slot_token, counts,
                offsets, toff, meta, p.E, p.H, p.I, nt_dn, S);
    return hipGetLastError();
  }
  BEAM_LAUNCH(tm, "gate_up_fp8", grouped_gemm_fp8<kGateUp>, grid_for(p, nt_gu),
              dim3(kThreads), 0, s, xq, xss, w_gate_up, s_gate_up, hq, hs, slot_token,
              counts, offsets, toff, meta, p.E, p.H, p.I, nt_gu, p.xt, S);
  BEAM_LAUNCH(tm, "down_fp8", grouped_gemm_fp8<kDown>, grid_for(p, nt_dn),
              dim3(kThreads), 0, s, hq, hs, w_down, s_down, y, nullptr, slot_token,
              counts, offsets, toff, meta, p.E, p.H, p.I, nt_dn, p.xt, S);
  return hipGetLastError();
}

}  // namespace beam
