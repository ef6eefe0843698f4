// Weighted combine of the K expert outputs of each token: out[t] =
// sum_k w[t,k] y[slot(t,k)], accumulated in fp32 in rank order and rounded
// once to the output dtype.  There is no shared expert to add ("Reflection
// Releases Beam ...", section "Where Beam Saves and Where the Memory Bill
// Comes In").  8 consecutive columns per thread.
//
// combine_residual also applies the step after the block: the post-sublayer
// RMSNorm of SandwichNorm and the depth-scaled FP32 residual stream
// ("Reflection Beam", section "Hybrid Attention and Unusual Residuals";
// pretraining paragraph of "Reflection AI Introduces Beam ..."):
//   r = sqrt((k-1)/k) r + (1/sqrt(k)) o / sqrt(mean(o^2) + eps) * gamma
// on the fp32 block output o before any rounding, held in LDS between the
// two passes; the sum of squares is reduced in a fixed order.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float* v);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4 q = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __uint_as_float(a[i]);
    v[4 + i] = __uint_as_float(b[i]);
  }
}

template <typename YT>
__device__ __forceinline__ void store_out(void* out, int64_t at, const float* acc, bool bf16) {
  if (bf16) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      q[i] = static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i + 1])) << 16);
    st16(static_cast<uint16_t*>(out) + at, q);
  } else {
    float* o = static_cast<float*>(out) + at;
    st16(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                  __float_as_uint(acc[2]), __float_as_uint(acc[3])});
    st16(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                      __float_as_uint(acc[6]), __float_as_uint(acc[7])});
  }
}

// Columns c .. c + 7 of token t.
template <typename YT, bool OUT_BF16, int KM>
__device__ __forceinline__ void combine_cols(const YT* __restrict__ y,
                                             const int32_t* __restrict__ slot_of,
                                             const float* __restrict__ w, void* __restrict__ out,
                                             int K, int H, int64_t t, int c) {
  constexpr int kMaxK = KM;
  float v[kMaxK][8];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k)
    if (k < K) load8<YT>(y + static_cast<int64_t>(slot_of[t * K + k]) * H + c, v[k]);
  float acc[8] = {};
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k < K) {
      const float wk = w[t * K + k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wk, v[k][i], acc[i]);
    }
  }
  if (OUT_BF16) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      q[i] = static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i + 1])) << 16);
    st16(static_cast<uint16_t*>(out) + t * H + c, q);
  } else {
    float* o = static_cast<float*>(out) + t * H + c;
    st16(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                  __float_as_uint(acc[2]), __float_as_uint(acc[3])});
    st16(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                      __float_as_uint(acc[6]), __float_as_uint(acc[7])});
  }
}

// Workgroup (t, j) sums token t's columns 1024 j .. 1024 j + 1023 (a decode
// batch still fills the chip), with the K rows' loads all issued before the
// sums (which run in rank order).  KM bounds K: 8 holds the loads in 64
// registers per thread, 16 in 128.
template <typename YT, bool OUT_BF16, int KM>
__global__ __launch_bounds__(128) void combine_split(
    const YT* __restrict__ y, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, void* __restrict__ out, int K, int H) {
  const int c = (blockIdx.y * 128 + threadIdx.x) * 8;
  if (c < H) combine_cols<YT, OUT_BF16, KM>(y, slot_of, w, out, K, H, blockIdx.x, c);
}

// K > 8 on large batches: one workgroup per token, the same sums column
// group by column group (fewer registers per thread than combine_split<16>).
template <typename YT, bool OUT_BF16>
__global__ __launch_bounds__(128) void combine(
    const YT* __restrict__ y, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, void* __restrict__ out, int K, int H) {
  const int64_t t = blockIdx.x;
  int slot[16];
  float wk[16];
  for (int k = 0; k < K; ++k) {
    slot[k] = slot_of[t * K + k];
    wk[k] = w[t * K + k];
  }
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8] = {};
    for (int k = 0; k < K; ++k) {
      float v[8];
      load8<YT>(y + static_cast<int64_t>(slot[k]) * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wk[k], v[i], acc[i]);
    }
    store_out<YT>(out, t * H + c, acc, OUT_BF16);
  }
}


constexpr int kCombineThreads = 128;

template <typename YT, bool OUT_BF16>
__global__ __launch_bounds__(kCombineThreads) void combine_residual(
    const YT* __restrict__ y, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, void* __restrict__ out, int K, int H,
    const float* __restrict__ gamma, float eps, float a, float b,
    float* __restrict__ residual) {
  extern __shared__ float row[];  // the token's fp32 block output, H values
  __shared__ float part[kCombineThreads / kWave];
  const int64_t t = blockIdx.x;
  int slot[16];
  float wk[16];
  for (int k = 0; k < K; ++k) {
    slot[k] = slot_of[t * K + k];
    wk[k] = w[t * K + k];
  }
  float ss = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += kCombineThreads * 8) {
    float acc[8] = {};
    for (int k = 0; k < K; ++k) {
      float v[8];
      load8<YT>(y + static_cast<int64_t>(slot[k]) * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wk[k], v[i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      row[c + i] = acc[i];
      ss = __builtin_fmaf(acc[i], acc[i], ss);
    }
    if (out) store_out<YT>(out, t * H + c, acc, OUT_BF16);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / kWave; ++i) total += part[i];
  const float inv = 1.0f / sqrtf(total / static_cast<float>(H) + eps);
  for (int c = threadIdx.x * 8; c < H; c += kCombineThreads * 8) {
    float* r = residual + t * H + c;
    const u32x4 r0 = ld16(r), r1 = ld16(r + 4);
    const u32x4 g0 = ld16(gamma + c), g1 = ld16(gamma + c + 4);
    float nr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float rv = __uint_as_float(i < 4 ? r0[i] : r1[i - 4]);
      const float gv = __uint_as_float(i < 4 ? g0[i] : g1[i - 4]);
      const float n = row[c + i] * inv * gv;
      nr[i] = __builtin_fmaf(a, rv, b * n);
    }
    st16(r, u32x4{__float_as_uint(nr[0]), __float_as_uint(nr[1]), __float_as_uint(nr[2]),
                  __float_as_uint(nr[3])});
    st16(r + 4, u32x4{__float_as_uint(nr[4]), __float_as_uint(nr[5]), __float_as_uint(nr[6]),
                      __float_as_uint(nr[7])});
  }
}

}  // namespace

hipError_t launch_combine(const Plan& p, const int32_t* slot_of,
                          const float* w, void* out, void* ws, hipStream_t s,
                          Timer* tm, const Epilogue* ep) {
  const dim3 grid(static_cast<unsigned>(p.T)), block(128);
  // combine_split for K <= 8 at every T (16K tokens: 0.30 ms against 0.32
  // for one workgroup per token; 8K fp8: 0.154 against 0.166); for larger K
  // only below 2K tokens (64 tokens: 23 -> under 20 us), as with 16 rows'
  // loads in flight it took 0.36 ms at 16K against 0.30 for combine
  const bool split = p.T < 2048;
  const dim3 grid_cols(static_cast<unsigned>(p.T), static_cast<unsigned>(ceil_div(p.H, 1024)));
  const bool y_f32 = p.wdt == BEAM_F32 || p.wdt == BEAM_MXFP4 || p.stream_path;
  const bool out_bf16 = p.act == BEAM_BF16;
  if (ep) {
    const size_t lds = static_cast<size_t>(p.H) * sizeof(float);
#define BEAM_COMBINE_RES(YT, OB, YP)                                                        \
  BEAM_LAUNCH(tm, "combine_residual", (combine_residual<YT, OB>), grid, dim3(kCombineThreads), \
              lds, s, YP, slot_of, w, out, p.K, p.H, ep->gamma, ep->eps, ep->a, ep->b,       \
              ep->residual)
    if (y_f32) {
      const float* y = ws_at<float>(ws, p.off_y);
      if (out_bf16) BEAM_COMBINE_RES(float, true, y); else BEAM_COMBINE_RES(float, false, y);
    } else {
      const uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
      if (out_bf16) BEAM_COMBINE_RES(uint16_t, true, y); else BEAM_COMBINE_RES(uint16_t, false, y);
    }
#undef BEAM_COMBINE_RES
    return hipGetLastError();
  }
#define BEAM_COMBINE(YT, OB, YP)                                                             \
  do {                                                                                       \
    if (p.K <= 8)                                                                            \
      BEAM_LAUNCH(tm, "combine", (combine_split<YT, OB, 8>), grid_cols, block, 0, s, YP, slot_of, \
                  w, out, p.K, p.H);                                                         \
    else if (split)                                                                          \
      BEAM_LAUNCH(tm, "combine", (combine_split<YT, OB, 16>), grid_cols, block, 0, s, YP, slot_of, \
                  w, out, p.K, p.H);                                                         \
    else                                                                                     \
      BEAM_LAUNCH(tm, "combine", (combine<YT, OB>), grid, block, 0, s, YP, slot_of, w, out,   \
                  p.K, p.H);                                                                 \
  } while (0)
  if (y_f32) {
    const float* y = ws_at<float>(ws, p.off_y);
    if (out_bf16) BEAM_COMBINE(float, true, y); else BEAM_COMBINE(float, false, y);
  } else {
    const uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
    if (out_bf16) BEAM_COMBINE(uint16_t, true, y); else BEAM_COMBINE(uint16_t, false, y);
  }
#undef BEAM_COMBINE
  return hipGetLastError();
}

}  // namespace beam
