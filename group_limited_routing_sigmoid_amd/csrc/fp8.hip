// FP8 (OCP e4m3fn) variant of the expert path.  The pages name FP8
// checkpoints ("Hugging Face releases Beam ..." checkpoint paragraph;
// "Reflection Beam", section "Where to run it") without a recipe; this
// library reads it as e4m3fn weights with one fp32 scale per 128x128 block,
// activations quantised per token per 128 channels with scale = amax/448,
// and fp32 accumulation with the scales applied per 128-deep slice.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

// binary32 -> e4m3fn, round to nearest even, magnitudes >= 448 saturate.
__device__ __forceinline__ uint32_t e4m3_rne(float f) {
  const uint32_t bits = __float_as_uint(f);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;            // NaN
  const float a = __uint_as_float(mag);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                                   // below 2^-6: step 2^-9
    return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  }
  int ex = static_cast<int>(mag >> 23) - 127;            // -6 .. 8
  uint32_t keep = (mag >> 20) & 7u;
  const uint32_t rest = mag & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0;
    ++ex;
  }
  uint32_t code = (static_cast<uint32_t>(ex + 7) << 3) | keep;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// One wave per (row, 128-column block); lane i handles columns 2i, 2i+1.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_e4m3_rows(
    const void* __restrict__ v, int64_t rows, int64_t cols,
    uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int lane = threadIdx.x % kWave;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int64_t nbc = cols / 128;
  if (blk >= rows * nbc) return;
  const int64_t r = blk / nbc, c = (blk % nbc) * 128 + 2 * lane;
  float a0, a1;
  if (BF16) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(
        static_cast<const uint16_t*>(v) + r * cols + c);
    a0 = __uint_as_float(pair << 16);
    a1 = __uint_as_float(pair & 0xFFFF0000u);
  } else {
    const float* p = static_cast<const float*>(v) + r * cols + c;
    a0 = p[0];
    a1 = p[1];
  }
  float m = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float sc = (m > 0.0f) ? m / 448.0f : 1.0f;
  const uint32_t c0 = e4m3_rne(a0 / sc), c1 = e4m3_rne(a1 / sc);
  *reinterpret_cast<uint16_t*>(q + r * cols + c) = static_cast<uint16_t>(c0 | (c1 << 8));
  if (lane == 0) scales[blk] = sc;
}

}  // namespace

hipError_t launch_quant_e4m3(int64_t rows, int64_t cols, int32_t dtype,
                             const void* v, uint8_t* q, float* scales,
                             hipStream_t s, Timer* tm) {
  const int64_t blocks = rows * (cols / 128);
  const dim3 grid(static_cast<unsigned>(ceil_div(blocks, 4)));
  if (dtype == BEAM_BF16)
    BEAM_LAUNCH(tm, "quant_e4m3", quant_e4m3_rows<true>, grid, dim3(256), 0, s, v, rows, cols, q, scales);
  else
    BEAM_LAUNCH(tm, "quant_e4m3", quant_e4m3_rows<false>, grid, dim3(256), 0, s, v, rows, cols, q, scales);
  return hipGetLastError();
}

bool fp8_experts_built() { return true; }

namespace {

constexpr int BM = kGemmBM;  // 256 slots
constexpr int BN = 128;
constexpr int BK = 128;      // one scale block per k step
constexpr int kThreads = 512;
constexpr int kRowBytes = BK;                // 128 e4m3 codes per tile row
constexpr int kATile = BM * kRowBytes;       // 32 KiB
constexpr int kBTile = BN * kRowBytes;       // 16 KiB
constexpr int kXcds = 8;
constexpr int kALoads = kATile / (16 * kThreads);  // 4
constexpr int kBLoads = kBTile / (16 * kThreads);  // 2

enum Mode { kGateUp = 0, kDown = 1 };

__device__ __forceinline__ int swz(int row, int chunk) {
  // the 8 chunks of any 8 consecutive rows land on distinct bank groups,
  // and so do the even (and the odd) rows of any 16 consecutive rows
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int n_nt, int L) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] * n_nt <= L) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// D = A(32x64) * B(64x32) + C on e4m3 codes (format 0, unit E8M0 scales).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Grouped e4m3 GEMM with per-128 block scales: for every 128-deep slice kb,
// P = sum_k qa*qw on the matrix cores (exact products, fp32 sums), then
// acc += P * (s_a[row, kb] * s_w[nblock, kb]) in fp32.  Same work list, XCD
// order and SwiGLU epilogue as the bf16 grouped GEMM; 256x128 tiles (a
// gate/up tile = 64 gate + 64 up rows), 8 waves of 64x64, LDS double buffer.
template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8(
    const uint8_t* __restrict__ a_src,   // gate/up: xq [T,H]; down: hq [S,I]
    const float* __restrict__ a_scale,   // gate/up: xs [T,H/128]; down: hs [S,I/128]
    const uint8_t* __restrict__ w,       // W_gu [E,2I,H] or W_d [E,H,I] codes
    const float* __restrict__ w_scale,   // [E,2I/128,H/128] or [E,H/128,I/128]
    uint16_t* __restrict__ out,          // gate/up: h [S,I] bf16; down: y [S,H] bf16
    const int32_t* __restrict__ slot_token, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ meta, int E, int H, int I, int n_nt) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kATile + kBTile];
  __shared__ __attribute__((aligned(16))) float sa[2][BM];

  const int n_log = meta[kMetaTiles] * n_nt;
  const int per_xcd = (n_log + kXcds - 1) / kXcds;
  const int local = blockIdx.x / kXcds;
  const int L = (blockIdx.x % kXcds) * per_xcd + local;
  if (local >= per_xcd || L >= n_log) return;
  const int e = find_expert(tile_off, E, n_nt, L);
  const int t0 = tile_off[e], nt_e = tile_off[e + 1] - t0;
  const int j = L - t0 * n_nt;
  const int nt = j / nt_e;
  const int row0 = offsets[e] + (j % nt_e) * BM;
  const int row_end = offsets[e] + counts[e];
  const int K = (MODE == kGateUp) ? H : I;
  const int nkb = K / 128;

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  const int chunk = tid % 8;
  const uint8_t* wbase = (MODE == kGateUp) ? w + static_cast<int64_t>(e) * 2 * I * H
                                           : w + static_cast<int64_t>(e) * H * I;
  uint32_t a_off[kALoads], b_off[kBLoads];
  int la_off[kALoads], lb_off[kBLoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r = tid / 8 + (kThreads / 8) * i;
    int slot = row0 + r;
    if (slot > row_end - 1) slot = row_end - 1;
    a_off[i] = (MODE == kGateUp) ? static_cast<uint32_t>(slot_token[slot]) * H + chunk * 16
                                 : static_cast<uint32_t>(slot) * I + chunk * 16;
    la_off[i] = swz(r, chunk);
  }
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int r = tid / 8 + (kThreads / 8) * i;
    if (MODE == kGateUp) {
      // rows 0..63: gate channels nt*64 + r; rows 64..127: up channels
      const int wrow = (r < 64) ? (nt * 64 + r) : (I + nt * 64 + (r - 64));
      b_off[i] = static_cast<uint32_t>(wrow) * H + chunk * 16;
    } else {
      b_off[i] = static_cast<uint32_t>(nt * BN + r) * I + chunk * 16;
    }
    lb_off[i] = kATile + swz(r, chunk);
  }
  // row scale source for threads 0..255 (one A row each)
  uint32_t sa_off = 0;
  if (tid < BM) {
    int slot = row0 + tid;
    if (slot > row_end - 1) slot = row_end - 1;
    sa_off = (MODE == kGateUp) ? static_cast<uint32_t>(slot_token[slot]) * nkb
                               : static_cast<uint32_t>(slot) * nkb;
  }
  // weight-scale rows of this wave's two 32-column blocks
  const float* sw0;
  const float* sw1;
  if (MODE == kGateUp) {
    const int cb = (nt * 64) / 128;  // 128-channel block of this tile's channels
    sw0 = w_scale + (static_cast<int64_t>(e) * (2 * I / 128) + cb) * nkb;
    sw1 = w_scale + (static_cast<int64_t>(e) * (2 * I / 128) + I / 128 + cb) * nkb;
  } else {
    sw0 = w_scale + (static_cast<int64_t>(e) * (H / 128) + nt) * nkb;
    sw1 = sw0;
  }

  u32x4 ra[kALoads], rb[kBLoads];
  float rs = 0.0f;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kALoads; ++i) ra[i] = ld16(a_src + (a_off[i] + kb * 128));
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) rb[i] = ld16(wbase + (b_off[i] + kb * 128));
    if (tid < BM) rs = a_scale[sa_off + kb];
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kALoads; ++i) *reinterpret_cast<u32x4*>(&lds[buf][la_off[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) *reinterpret_cast<u32x4*>(&lds[buf][lb_off[i]]) = rb[i];
    if (tid < BM) sa[buf][tid] = rs;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[i][n] = f32x16{};

  // A rows of this wave: wm*64 + i*32 + lane%32.  B rows: gate/up -> gate
  // wn*32 + lane%32, up 64 + wn*32 + lane%32; down -> wn*64 + n*32 + lane%32.
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) arow[i] = wm * 64 + i * 32 + lane % 32;
#pragma unroll
  for (int n = 0; n < 2; ++n)
    brow[n] = (MODE == kGateUp) ? (n * 64 + wn * 32 + lane % 32)
                                : (wn * 64 + n * 32 + lane % 32);

  // lane's 32 codes of a 64-deep half: chunks hlf*4 + 2*(lane/32) and +1
  auto frag = [&](int buf, int base, int row, int hlf) {
    const int c = hlf * 4 + 2 * (lane / 32);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(&lds[buf][base + swz(row, c)]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(&lds[buf][base + swz(row, c + 1)]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  auto compute = [&](int buf, int kb) {
    const float w0 = sw0[kb], w1 = sw1[kb];
    i32x8 a[2][2], b[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i][0] = frag(buf, 0, arow[i], 0);
      a[i][1] = frag(buf, 0, arow[i], 1);
      b[i][0] = frag(buf, kATile, brow[i], 0);
      b[i][1] = frag(buf, kATile, brow[i], 1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x16 p = {};
        p = mfma_fp8_32x32x64(a[i][0], b[n][0], p);
        p = mfma_fp8_32x32x64(a[i][1], b[n][1], p);
        const float wsc = n == 0 ? w0 : w1;
        // element r of p is row wm*64 + i*32 + 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(
              &sa[buf][wm * 64 + i * 32 + 8 * q + 4 * (lane / 32)]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[i][n][4 * q + t] = __builtin_fmaf(p[4 * q + t], v[t] * wsc, acc[i][n][4 * q + t]);
        }
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    compute(buf, kb);
    if (kb + 1 < nkb) sstore(buf ^ 1);
    __syncthreads();
  }

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
        for (int n = 0; n < 2; ++n) {
          const int col = nt * BN + wn * 64 + n * 32 + lane % 32;
          out[static_cast<int64_t>(row) * H + col] = f32_to_bf16_bits(acc[i][n][r]);
        }
      }
    }
  }
}

}  // namespace

// x -> e4m3 (per token, per 128 channels); gate/up GEMM with SwiGLU -> h
// (bf16); h -> e4m3 (per slot, per 128 channels); down GEMM -> y (bf16).
hipError_t launch_experts_fp8(const Plan& p, const void* x,
                              const uint8_t* w_gate_up, const float* s_gate_up,
                              const uint8_t* w_down, const float* s_down,
                              void* ws, hipStream_t s, Timer* tm) {
  uint8_t* xq = ws_at<uint8_t>(ws, p.off_xq);
  float* xs = ws_at<float>(ws, p.off_xs);
  uint8_t* hq = ws_at<uint8_t>(ws, p.off_hq);
  float* hs = ws_at<float>(ws, p.off_hs);
  uint16_t* h = ws_at<uint16_t>(ws, p.off_h);
  uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* toff = ws_at<int32_t>(ws, p.off_tile_off);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  hipError_t e = launch_quant_e4m3(p.T, p.H, BEAM_BF16, x, xq, xs, s, tm);
  if (e != hipSuccess) return e;
  const int nt_gu = p.I / 64, nt_dn = p.H / BN;
  auto grid_for = [&](int n_nt) {
    const int64_t per = ceil_div(p.max_tiles * n_nt, kXcds);
    return dim3(static_cast<unsigned>(per * kXcds));
  };
  BEAM_LAUNCH(tm, "gate_up_fp8", grouped_gemm_fp8<kGateUp>, grid_for(nt_gu),
              dim3(kThreads), 0, s, xq, xs, w_gate_up, s_gate_up, h, slot_token,
              counts, offsets, toff, meta, p.E, p.H, p.I, nt_gu);
  e = launch_quant_e4m3(p.S, p.I, BEAM_BF16, h, hq, hs, s, tm);
  if (e != hipSuccess) return e;
  BEAM_LAUNCH(tm, "down_fp8", grouped_gemm_fp8<kDown>, grid_for(nt_dn),
              dim3(kThreads), 0, s, hq, hs, w_down, s_down, y, slot_token,
              counts, offsets, toff, meta, p.E, p.H, p.I, nt_dn);
  return hipGetLastError();
}

}  // namespace beam
