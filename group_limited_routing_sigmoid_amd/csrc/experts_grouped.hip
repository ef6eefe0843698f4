// Expert MLPs as grouped matrix products on the gfx950 matrix cores (bf16
// inputs, fp32 sums), for batches where each expert sees many tokens.
//
// Each expert is a SwiGLU MLP, hidden 5,120 -> intermediate 2,560 -> hidden
// ("Hugging Face releases Beam ..." MoE paragraph; "Reflection Releases Beam
// ...", section "Where Beam Saves and Where the Memory Bill Comes In"):
//   gate/up  h[slot, c] = silu(x[tok] . W_gu[e, c]) * (x[tok] . W_gu[e, I+c])
//   down     y[slot, n] = h[slot] . W_d[e, n]
// Work is a list of (expert, 128-slot M tile) entries built by the
// permutation kernels, crossed with N tiles.  A gate/up tile holds 64 gate
// and the matching 64 up rows of W_gu, so one wave owns both halves of its
// channels and applies silu(g)*u in registers; x rows are gathered by slot
// inside the A loads, so no permuted copy of x is made.  Tiles are staged in
// LDS (double buffered, 16-byte chunks XOR-swizzled by row), and each wave
// computes 64x64 with 32x32x16 bf16 MFMA.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

constexpr int BM = kGemmBM;  // 128 slots
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK * 2;  // 128 bytes per tile row in LDS
constexpr int kTileBytes = BM * kRowBytes;

enum Mode { kGateUp = 0, kDown = 1 };

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// grid: max_tiles * n_tiles; block 256.
template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(
    const uint16_t* __restrict__ a_src,   // gate/up: x [T,H]; down: h [S,I]
    const uint16_t* __restrict__ w,       // W_gu [E,2I,H] or W_d [E,H,I]
    uint16_t* __restrict__ out,           // gate/up: h [S,I]; down: y [S,H]
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ meta,
    int H, int I, int n_tiles_n) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2 * kTileBytes];
  const int mt = blockIdx.x / n_tiles_n;
  const int nt = blockIdx.x % n_tiles_n;
  if (mt >= meta[kMetaTiles]) return;
  const int e = tile_expert[mt];
  const int row0 = tile_row0[mt];
  const int row_end = offsets[e] + counts[e];  // first slot past this expert
  const int K = (MODE == kGateUp) ? H : I;
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // --- global source rows for this thread's four A and four B chunks ------
  const int chunk = tid % 8;
  const uint16_t* a_ptr[4];
  const uint16_t* b_ptr[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tid / 8 + 32 * i;
    int slot = row0 + r;
    if (slot > row_end - 1) slot = row_end - 1;   // padded rows: any valid row
    if (MODE == kGateUp) {
      a_ptr[i] = a_src + static_cast<int64_t>(slot_token[slot]) * H + chunk * 8;
      // rows 0..63: gate channels nt*64+r; rows 64..127: up channels
      const int wrow = (r < 64) ? (nt * 64 + r) : (I + nt * 64 + (r - 64));
      b_ptr[i] = w + (static_cast<int64_t>(e) * 2 * I + wrow) * H + chunk * 8;
    } else {
      a_ptr[i] = a_src + static_cast<int64_t>(slot) * I + chunk * 8;
      b_ptr[i] = w + (static_cast<int64_t>(e) * H + nt * BN + r) * I + chunk * 8;
    }
    lds_off[i] = swz(r, chunk);
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(a_ptr[i] + k0);
      rb[i] = ld16(b_ptr[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&lds[buf][lds_off[i]]) = ra[i];
      *reinterpret_cast<u32x4*>(&lds[buf][kTileBytes + lds_off[i]]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // A rows of this wave: wm*64 + mi*32 + lane%32.
  // B rows: gate/up -> gate wn*32 + lane%32 and up 64 + wn*32 + lane%32;
  //         down    -> wn*64 + ni*32 + lane%32.
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = wm * 64 + i * 32 + lane % 32;
    brow[i] = (MODE == kGateUp) ? (i * 64 + wn * 32 + lane % 32)
                                : (wn * 64 + i * 32 + lane % 32);
  }

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + lane / 32;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&lds[buf][swz(arow[i], c)]));
        bfr[i] = as_bf16x8(
            *reinterpret_cast<const u32x4*>(&lds[buf][kTileBytes + swz(brow[i], c)]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue ------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      if (row >= row_end) continue;
      if (MODE == kGateUp) {
        const int ch = nt * 64 + wn * 32 + lane % 32;
        const float h = silu(acc[i][0][r]) * acc[i][1][r];
        out[static_cast<int64_t>(row) * I + ch] = f32_to_bf16_bits(h);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nt * BN + wn * 64 + j * 32 + lane % 32;
          out[static_cast<int64_t>(row) * H + n] = f32_to_bf16_bits(acc[i][j][r]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_bf16(const Plan& p, const void* x,
                               const void* w_gate_up, const void* w_down,
                               void* ws, hipStream_t s, Timer* tm) {
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* te = ws_at<int32_t>(ws, p.off_tile_expert);
  const int32_t* tr = ws_at<int32_t>(ws, p.off_tile_row0);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  uint16_t* h = ws_at<uint16_t>(ws, p.off_h);
  uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
  const int nt_gu = p.I / 64;
  const int nt_dn = p.H / BN;
  BEAM_LAUNCH(tm, "grouped_gate_up_bf16", grouped_gemm_bf16<kGateUp>,
                     dim3(static_cast<unsigned>(p.max_tiles * nt_gu)),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w_gate_up), h, slot_token,
                     counts, offsets, te, tr, meta, p.H, p.I, nt_gu);
  BEAM_LAUNCH(tm, "grouped_down_bf16", grouped_gemm_bf16<kDown>,
                     dim3(static_cast<unsigned>(p.max_tiles * nt_dn)),
                     dim3(kThreads), 0, s, h,
                     static_cast<const uint16_t*>(w_down), y, slot_token,
                     counts, offsets, te, tr, meta, p.H, p.I, nt_dn);
  return hipGetLastError();
}

}  // namespace beam
