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
// Work is the list of (expert, M tile) entries built by the permutation
// kernels, crossed with 256-wide N tiles.  A gate/up N tile holds 128 gate
// rows of W_gu and the 128 matching up rows, so every wave owns both halves
// of its channels and applies silu(g)*u in registers; x rows are gathered by
// slot inside the A loads (no permuted copy of x).  Tiles move from global
// memory straight into LDS, 16-byte chunks XOR-swizzled by row so the MFMA
// operand reads are bank-conflict free.  256-row tiles: four waves of
// 128x128 (below); 128- and 160-row tiles for experts holding few rows:
// eight waves with a three-stage copy ring (further below).
//
// Tile layout, DMA pattern and the XCD-aware tile order: grouped_tile.h.
//
// Router logits for many tokens use the same tile loop as a dense product:
// the fp32 router matrix is split exactly into three bf16 matrices, laid side
// by side along k (W3 [E, 3H]) and multiplied with x repeated three times
// (its column index wraps modulo H), so every product is exact and the sums
// are fp32.  The reduction is split into ks slices; the router's selection
// kernel adds the ks partial logits in a fixed order.
#include <utility>

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

// ---- 256 x 256 tiles, four waves of 128 x 128 ---------------------------------
// For batches whose experts reuse their weights over several M tiles.  One
// wave per SIMD, each wave 128 rows x 128 columns: its 256 fp32 sums stay in
// the accumulation registers, and a stage's fragment reads from LDS are
// 128 KiB per workgroup (two thirds of the eight-wave layout's).  Wave (wm,
// wn) takes the 32-row A fragments 2f + wm (f = 0..3), so a partial tile's
// valid rows split evenly over the two SIMD halves; its B rows are gate rows
// 64 wn .. +63 with the matching up rows 128 + 64 wn .. +63 (gate/up), or
// rows 128 wn .. +127 (down).  Stages are 64 deep (same tile layout and
// swizzle as the other forms), copied straight into LDS: token (or h) rows
// double buffered, weight rows triple buffered, so the weight copies go out
// about 1.75 stages before they are read (mainloop4).
// The wave's instruction stream is ordered by hand (scheduling fences after
// every product): a wave issues in order, so a burst of memory instructions
// between bursts of products leaves its SIMD's matrix core idle while it
// issues them; one memory instruction after each product keeps it fed.  The
// stage boundary sits inside the last k16 step: half of its products are
// issued, the wave waits for its LDS traffic and meets the others, then
// reads the next stage's first fragments between the other half.  Same
// products in the same k order as the other tile forms: bit-identical.
namespace w4 {

constexpr int kThreads4 = 256;

// Two floats to two bf16 (round to nearest even, as f32_to_bf16_bits), x in
// the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float2 v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v.x, v.y}, bf16x2_t));
}
// The low (high) halves of a and b, a's in the low half of the result.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

// s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0) / lgkmcnt(0) alone (vmcnt 63 and
// expcnt 7 mean "no wait") / lgkmcnt(0) then s_barrier, as builtins so the
// compiler's wait-count tracking knows the counters afterwards (it cannot
// see into inline assembly).
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// lgkmcnt(8): all but this wave's last 8 LDS operations have completed
__device__ __forceinline__ void wait_lds_but8() { __builtin_amdgcn_s_waitcnt(0xC87F); }
__device__ __forceinline__ void wait_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

// Per-lane byte offsets, computed once per tile.  With the swizzle
// swz(row, chunk), a row's key (row ^ (row >> 3)) & 7 depends only on the
// lane and on the parity of the 32-row block (the 8-row region) the row
// lies in, so a few bases plus constants address every access.
struct Addr4 {
  uint32_t a_vo[8];     // global: this lane's A row and chunk, copy region i
  uint32_t b_vo[2];     // global: this lane's row and chunk inside a B region of parity p
  uint32_t b_so[8];     // global, wave-uniform: B region i's first row
  uint32_t a_rd[4];     // LDS, inside an A buffer: A fragment 0 of k16 step kk
  uint32_t b_rd[4][2];  // LDS, inside a B buffer: B fragment n of k16 step kk,
                        // n % 2 = p, less bimm(n)
};

// LDS byte offset of B fragment n beyond b_rd[.][n % 2]
template <int MODE>
__device__ __forceinline__ constexpr int bimm(int n) {
  return (MODE == kGateUp) ? (n / 2) * 16384 : (n / 2) * 8192;
}

struct Frags4 {
  bf16x8 a[4], b[4];
};

// Fragment read j of a k16 step: A fragment j (j < 4, rows 32 (2 j + wm))
// from the A buffer at LDS byte offset abuf, or B fragment j - 4 from the B
// buffer at bbuf.
template <int NF, int MODE>
__device__ __forceinline__ void read_frag(Frags4& f, int j, const unsigned char* L,
                                          uint32_t abuf, uint32_t bbuf, int kk,
                                          const Addr4& ad) {
  if (j < 4) {
    if (j < NF)
      f.a[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(L + abuf + ad.a_rd[kk] + j * 8192));
  } else {
    const int n = j - 4;
    f.b[n] = as_bf16x8(
        *reinterpret_cast<const u32x4*>(L + bbuf + ad.b_rd[kk][n & 1] + bimm<MODE>(n)));
  }
}

// Product j of a k16 step: A fragment j / 4 with B fragment j % 4.
template <int NF>
__device__ __forceinline__ void mfma_j(const Frags4& f, int j, f32x16 (&acc)[4][4]) {
  if (j / 4 < NF) acc[j / 4][j % 4] = mfma32x32x16(f.a[j / 4], f.b[j % 4], acc[j / 4][j % 4]);
}

// LDS of the four-wave tiles (160 KiB, all of it): two A buffers (token or
// h rows, 32 KiB each) and three B buffers (weight rows), so that the weight
// copies, which miss the caches most, can be issued two stages ahead.
constexpr int kLds4 = 5 * kTileBytes;
constexpr int kABuf0 = 0, kBBuf0 = 2 * kTileBytes;

// One 16-byte-per-lane copy straight into LDS (1 KiB per wave): region
// wave + 4 i of the A tile (A = true) or of the B tile, stage k, into the
// buffer at LDS byte offset buf.  Buffer loads with the LDS flag: the lane's
// 16 bytes land at M0 + 16 lane, M0 = the region's (wave-uniform) start.
template <bool A>
__device__ __forceinline__ void copy_i(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                       unsigned char* L, uint32_t buf, int k, int i,
                                       const Addr4& ad, int wave) {
  __attribute__((address_space(3))) void* dst =
      (__attribute__((address_space(3))) void*)(L + buf + (wave + 4 * i) * 1024);
  if (A)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, ad.a_vo[i], 2 * k, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, ad.b_vo[i & 1], ad.b_so[i] + 2 * k, 0,
                                             0);
}

// Stage t reads A buffer t % 2 and B buffer t % 3.  Its 64 products are
// slots 0..63 (k16 step s / 16), the barrier between slots 55 and 56.  A
// compute unit's texture path takes about 64 bytes a cycle, so the copies
// (64 KiB per stage per workgroup) are spread over the stage rather than
// issued in bursts (four waves issuing together in a window of a few
// products stall at issue):
// - token rows of stage t + 1, into A buffer (t + 1) % 2 (free since stage
//   t - 1's barrier): regions 0, 1 at slots 58, 62 of stage t - 1, regions
//   2..7 at slots 1, 4, .., 16 of stage t;
// - weights of stage t + 2, into B buffer (t + 2) % 3 (free since stage
//   t - 1's barrier): regions 0..7 at slots 20, 24, .., 48.
// Both must have landed by stage t + 1's barrier.  Every copy is a direct
// LDS load, so the copies complete in issue order and "stage t + 1 has
// landed" at stage t's barrier is vmcnt(8): only stage t + 2's 8 weight
// copies per wave were issued after the last of them.  (A load into
// registers may complete before an earlier copy into LDS, so the two kinds
// are never mixed here.)  Fragment reads: those of k16 step k + 1 in the
// first 8 slots of step k, those of the next stage's step 0 two per slot
// after the barrier.
// LDS offsets and k columns of one stage's slots
struct Stage4 {
  uint32_t ca, na;       // A buffers of stages t and t + 1
  uint32_t cb, nbb, b2;  // B buffers of stages t, t + 1 and t + 2
  int kn1, kn2;          // k columns of stages t + 1 and t + 2
};

// Slot S (a compile-time constant) of a stage: its product and the memory
// operations issued beside it.  TAIL: 0 for stages t < nk - 2; 1 for stage
// nk - 2 and 2 for stage nk - 1, which issue no copies past the last stage
// (so their barriers wait for every copy).
template <int NF, int MODE, int TAIL, int S>
__device__ __forceinline__ void slot4(Frags4& f0, Frags4& f1, f32x16 (&acc)[4][4],
                                      __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                      unsigned char* L, const Addr4& ad, int wave,
                                      const Stage4& g) {
  constexpr int step = S / 16, j = S % 16;
  if constexpr (j == 0) wait_lds();
  if constexpr (S == 56) {
    // this wave's copies of stage t + 1 have landed and its reads of stage t
    // are done (vmcnt(8) lgkmcnt(0), or vmcnt(0) in the last two stages);
    // then every wave's are
    __builtin_amdgcn_s_waitcnt(TAIL == 0 ? 0x0078 : 0x0070);
    __builtin_amdgcn_s_barrier();
  }
  if constexpr (step % 2 == 0) mfma_j<NF>(f0, j, acc);
  else mfma_j<NF>(f1, j, acc);
  if constexpr (step < 3 && j < 8) {
    if constexpr (step % 2 == 0) read_frag<NF, MODE>(f1, j, L, g.ca, g.cb, step + 1, ad);
    else read_frag<NF, MODE>(f0, j, L, g.ca, g.cb, step + 1, ad);
  }
  if constexpr (S >= 56 && S < 60 && TAIL < 2) {
    read_frag<NF, MODE>(f0, 2 * (S - 56), L, g.na, g.nbb, 0, ad);
    read_frag<NF, MODE>(f0, 2 * (S - 56) + 1, L, g.na, g.nbb, 0, ad);
  }
  if constexpr (S >= 1 && S <= 16 && (S - 1) % 3 == 0 && TAIL < 2)
    copy_i<true>(ra, rb, L, g.na, g.kn1, 2 + (S - 1) / 3, ad, wave);
  if constexpr (S >= 20 && S <= 48 && S % 4 == 0 && TAIL == 0)
    copy_i<false>(ra, rb, L, g.b2, g.kn2, (S - 20) / 4, ad, wave);
  if constexpr ((S == 58 || S == 62) && TAIL == 0)
    copy_i<true>(ra, rb, L, g.ca, g.kn2, (S - 58) / 4, ad, wave);
  __builtin_amdgcn_sched_barrier(0);
}

template <int NF, int MODE, int TAIL, int... S>
__device__ __forceinline__ void stage4(std::integer_sequence<int, S...>, Frags4& f0, Frags4& f1,
                                       f32x16 (&acc)[4][4], __amdgpu_buffer_rsrc_t ra,
                                       __amdgpu_buffer_rsrc_t rb, unsigned char* L,
                                       const Addr4& ad, int wave, const Stage4& g) {
  (slot4<NF, MODE, TAIL, S>(f0, f1, acc, ra, rb, L, ad, wave, g), ...);
}

// LDS buffers and k columns of stage t (b3 = t % 3)
__device__ __forceinline__ Stage4 stage_at(int t, int b3, int nk) {
  Stage4 g;
  g.ca = (t & 1) * kTileBytes;
  g.na = kTileBytes - g.ca;
  g.cb = kBBuf0 + b3 * kTileBytes;
  const int b3n = (b3 == 2) ? 0 : b3 + 1;
  g.nbb = kBBuf0 + b3n * kTileBytes;
  g.b2 = kBBuf0 + (b3n == 2 ? 0 : b3n + 1) * kTileBytes;
  g.kn1 = min(t + 1, nk - 1) * BK;
  g.kn2 = min(t + 2, nk - 1) * BK;
  return g;
}

template <int NF, int MODE>
__device__ __forceinline__ void mainloop4(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          int nk, unsigned char* L, const Addr4& ad,
                                          f32x16 (&acc)[4][4]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  Frags4 f0, f1;
  const int k1 = min(1, nk - 1) * BK;
  if constexpr (MODE == kGateUp) {
    // (the weights of stages 0 and 1 went out before, in the kernel)
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<true>(ra, rb, L, kABuf0, 0, i, ad, wave);
    copy_i<true>(ra, rb, L, kABuf0 + kTileBytes, k1, 0, ad, wave);
    copy_i<true>(ra, rb, L, kABuf0 + kTileBytes, k1, 1, ad, wave);
    // stage 0 landed (stage 1's weights too): all but the last 2 copies
    __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<true>(ra, rb, L, kABuf0, 0, i, ad, wave);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<false>(ra, rb, L, kBBuf0, 0, i, ad, wave);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<false>(ra, rb, L, kBBuf0 + kTileBytes, k1, i, ad, wave);
    copy_i<true>(ra, rb, L, kABuf0 + kTileBytes, k1, 0, ad, wave);
    copy_i<true>(ra, rb, L, kABuf0 + kTileBytes, k1, 1, ad, wave);
    // stage 0 landed: all but stage 1's 10 copies so far
    __builtin_amdgcn_s_waitcnt(0x007A);  // vmcnt(10) lgkmcnt(0)
  }
  wait_lds_barrier();
#pragma unroll
  for (int j = 0; j < 8; ++j) read_frag<NF, MODE>(f0, j, L, kABuf0, kBBuf0, 0, ad);
  constexpr auto kSlots = std::make_integer_sequence<int, 64>{};
  int b3 = 0;  // t % 3
  int t = 0;
  for (; t < nk - 2; ++t) {
    stage4<NF, MODE, 0>(kSlots, f0, f1, acc, ra, rb, L, ad, wave, stage_at(t, b3, nk));
    b3 = (b3 == 2) ? 0 : b3 + 1;
  }
  if (t == nk - 2) {
    stage4<NF, MODE, 1>(kSlots, f0, f1, acc, ra, rb, L, ad, wave, stage_at(t, b3, nk));
    b3 = (b3 == 2) ? 0 : b3 + 1;
    ++t;
  }
  stage4<NF, MODE, 2>(kSlots, f0, f1, acc, ra, rb, L, ad, wave, stage_at(t, b3, nk));
  wait_all();
}

template <int MODE>
__global__ __launch_bounds__(kThreads4) void grouped_gemm_bf16_w4(
    const uint16_t* __restrict__ a_src,   // gate/up: x [T,H]; down: h [S,I]
    const uint16_t* __restrict__ w,       // W_gu [E,2I,H] or W_d [E,H,I]
    uint16_t* __restrict__ out,           // gate/up: h [S,I]; down: y [S,H]
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ meta, int T, int E, int H, int I, int n_nt) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds4];
  Coords tc;
  if (!tile_coords(counts, offsets, tile_off, meta, E, n_nt, tc)) return;
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, row_end = tc.row_end;
  const int K = (MODE == kGateUp) ? H : I;
  const int lane = threadIdx.x % kWave, l32 = lane % 32, hi = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const uint16_t* wbase = (MODE == kGateUp) ? w + static_cast<int64_t>(e) * 2 * I * H
                                            : w + static_cast<int64_t>(e) * H * I;
  const int m_valid = min(BM, row_end - row0);
  // buffer resources: x (or h) and this expert's weight matrix; loads past
  // either return zeros (the down product's last N tile may pass H)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(
      a_src, (MODE == kGateUp) ? static_cast<uint32_t>(T) * H * 2
                               : static_cast<uint32_t>(row_end) * I * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(
      wbase, static_cast<uint32_t>((MODE == kGateUp) ? 2 * I * H : H * I) * 2);
  Addr4 ad;
  // copy regions of this wave: wave + 4 i (i < 8) of A and of B, 8 rows each
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r0 = 8 * (wave + 4 * i);
    const int wrow0 = (MODE == kGateUp) ? ((r0 < 128) ? nt * 128 + r0 : I + nt * 128 + (r0 - 128))
                                        : nt * BN + r0;
    ad.b_so[i] = static_cast<uint32_t>(wrow0) * K * 2;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // rows 8 (wave + 4 i) + lane / 8 with i % 2 = p: key (lane / 8) ^ (wave + 4 p)
    const int c = (lane % 8) ^ (((lane / 8) ^ (wave + 4 * p)) & 7);
    ad.b_vo[p] = (static_cast<uint32_t>(lane / 8) * K + c * 8) * 2;
  }
  // Gate/up: the token indices of the wave's A rows are loaded first, all
  // eight, then the weights of stages 0 and 1 are copied while they are in
  // flight, then the token rows' addresses are formed (the down product's
  // rows are its slots; it copies stage 0's rows first, mainloop4).  Copies
  // of A rows past the tile's last valid row read past the end of the buffer
  // (zeros, no memory traffic; their sums are never stored).
  uint32_t src_row[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = min(row0 + 8 * (wave + 4 * i) + lane / 8, row_end - 1);
    src_row[i] = (MODE == kGateUp) ? static_cast<uint32_t>(slot_token[slot])
                                   : static_cast<uint32_t>(slot);
  }
  const int nk = K / BK;
  if constexpr (MODE == kGateUp) {
    const int k1 = min(1, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<false>(ra, rb, lds, kBBuf0, 0, i, ad, wave);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_i<false>(ra, rb, lds, kBBuf0 + kTileBytes, k1, i, ad, wave);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(src_row[i]));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (wave + 4 * i) + lane / 8;
    const int c = dma_chunk(r, lane);
    ad.a_vo[i] = (r < m_valid) ? (src_row[i] * ((MODE == kGateUp) ? H : I) + c * 8) * 2
                               : 0x80000000u;
  }
  const int key_a = ((lane & 7) ^ ((4 * wm + l32 / 8) & 7)) & 7;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ad.a_rd[kk] = (32 * wm + l32) * kRowBytes + ((((2 * kk + hi) ^ key_a) & 7) << 4);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key_b = ((lane & 7) ^ ((4 * p + l32 / 8) & 7)) & 7;
      const int rowb = ((MODE == kGateUp) ? wn * 64 : wn * 128) + p * 32 + l32;
      ad.b_rd[kk][p] = rowb * kRowBytes + ((((2 * kk + hi) ^ key_b) & 7) << 4);
    }
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[f][n] = f32x16{};
  // this wave's fragments holding a valid row: 2f + wm < ceil(m_valid / 32)
  const int g = (m_valid + 31) / 32;
  const int nf = min(4, max(0, (g - wm + 1) / 2));
  unsigned char* L = lds;
  switch (nf) {
    case 4: mainloop4<4, MODE>(ra, rb, nk, L, ad, acc); break;
    case 3: mainloop4<3, MODE>(ra, rb, nk, L, ad, acc); break;
    case 2: mainloop4<2, MODE>(ra, rb, nk, L, ad, acc); break;
    case 1: mainloop4<1, MODE>(ra, rb, nk, L, ad, acc); break;
    default: mainloop4<0, MODE>(ra, rb, nk, L, ad, acc); break;
  }
  // Epilogue through LDS: each lane holds 16 rows of one column, so the wave
  // writes its output tile (bf16) to its own LDS region first and stores it
  // back as 16-byte row pieces.  Every wave has finished reading the last
  // stage once all have passed the barrier.
  __builtin_amdgcn_s_barrier();
  constexpr int kCols = (MODE == kGateUp) ? 64 : 128;  // output columns per wave
  // LDS layout: pairs of rows interleaved, one 32-bit word per (row pair,
  // column) holding the even row's value in its low half and the odd row's
  // in its high half (a lane's rows 4q + 0..3 are two such pairs of one
  // column, so it writes both with one conversion and one 4-byte store);
  // pair pitch padded by 16 bytes on gate/up, the down product's 4 x 64
  // pairs of 512 bytes fill the stage buffers exactly
  constexpr int kPairPitch = (MODE == kGateUp) ? 4 * kCols + 16 : 4 * kCols;
  static_assert(4 * 64 * kPairPitch <= kLds4, "epilogue tile fits");
  unsigned char* R = L + wave * (64 * kPairPitch);
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (f >= nf) continue;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int pr = 16 * f + 4 * (r / 4) + 2 * hi + (r % 4) / 2;  // pair inside the wave's 64
#pragma unroll
      for (int n = 0; n < ((MODE == kGateUp) ? 2 : 4); ++n) {
        float2 v;
        if (MODE == kGateUp) {
          v.x = silu(acc[f][n][r]) * acc[f][n + 2][r];
          v.y = silu(acc[f][n][r + 1]) * acc[f][n + 2][r + 1];
        } else {
          v.x = acc[f][n][r];
          v.y = acc[f][n][r + 1];
        }
        *reinterpret_cast<uint32_t*>(R + pr * kPairPitch + 4 * (n * 32 + l32)) = pack_bf16x2(v);
      }
    }
  }
  wait_lds();
  // 16-byte row pieces, kPc per row: lane l takes piece l % kPc of the row
  // pairs l / kPc + kPairsPer i (two 16-byte reads give the piece of both
  // rows), so its column is fixed and every step's addresses are a constant
  // apart (the loop unrolls fully and the reads go out ahead of the stores)
  constexpr int kPc = kCols / 8;
  constexpr int kPairsPer = kWave / kPc;
  constexpr int kSteps = 64 / kPairsPer;
  const int pc = lane % kPc, pr0 = lane / kPc;
  const int col = ((MODE == kGateUp) ? nt * 128 + wn * 64 : nt * BN + wn * 128) + 8 * pc;
  const int ld = (MODE == kGateUp) ? I : H;
  const bool col_ok = col < ld;
  const unsigned char* rd = R + pr0 * kPairPitch + 32 * pc;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int pr = pr0 + kPairsPer * i;
    const int f = (kPairsPer * i) / 16;  // the A fragment these rows belong to
    const int row = row0 + 32 * (2 * f + wm) + 2 * (pr % 16);
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(rd + kPairsPer * i * kPairPitch);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(rd + kPairsPer * i * kPairPitch + 16);
    const u32x4 even = {lo_halves(w0[0], w0[1]), lo_halves(w0[2], w0[3]),
                        lo_halves(w1[0], w1[1]), lo_halves(w1[2], w1[3])};
    const u32x4 odd = {hi_halves(w0[0], w0[1]), hi_halves(w0[2], w0[3]),
                       hi_halves(w1[0], w1[1]), hi_halves(w1[2], w1[3])};
    if (f < nf && col_ok) {
      if (row < row_end) st16(out + static_cast<int64_t>(row) * ld + col, even);
      if (row + 1 < row_end) st16(out + static_cast<int64_t>(row + 1) * ld + col, odd);
    }
    if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // eight reads in flight at most
  }
}

}  // namespace w4

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
  BEAM_LAUNCH(tm, "grouped_gate_up_bf16", w4::grouped_gemm_bf16_w4<kGateUp>, grid_for(p, nt_gu),
              dim3(w4::kThreads4), 0, s, static_cast<const uint16_t*>(x),
              static_cast<const uint16_t*>(w_gate_up), h, slot_token, counts,
              offsets, toff, meta, static_cast<int>(p.T), p.E, p.H, p.I, nt_gu);
  BEAM_LAUNCH(tm, "grouped_down_bf16", w4::grouped_gemm_bf16_w4<kDown>, grid_for(p, nt_dn),
              dim3(w4::kThreads4), 0, s, h, static_cast<const uint16_t*>(w_down), y,
              slot_token, counts, offsets, toff, meta, static_cast<int>(p.T), p.E, p.H, p.I,
              nt_dn);
  return hipGetLastError();
}

}  // namespace beam
