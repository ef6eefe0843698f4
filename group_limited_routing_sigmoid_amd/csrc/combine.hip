// Weighted combine of the K expert outputs of each token: out[t] =
// sum_k w[t,k] y[slot(t,k)], accumulated in fp32 in rank order and rounded
// once to the output dtype.  There is no shared expert to add ("Reflection
// Releases Beam ...", section "Where Beam Saves and Where the Memory Bill
// Comes In").  One workgroup per token, 8 consecutive columns per thread.
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
}

}  // namespace

hipError_t launch_combine(const Plan& p, const int32_t* slot_of,
                          const float* w, void* out, void* ws, hipStream_t s,
                          Timer* tm) {
  const dim3 grid(static_cast<unsigned>(p.T)), block(128);
  const bool y_f32 = p.wdt == BEAM_F32 || p.stream_path;
  const bool out_bf16 = p.act == BEAM_BF16;
  if (y_f32) {
    const float* y = ws_at<float>(ws, p.off_y);
    if (out_bf16)
      BEAM_LAUNCH(tm, "combine", (combine<float, true>), grid, block, 0, s, y, slot_of, w, out, p.K, p.H);
    else
      BEAM_LAUNCH(tm, "combine", (combine<float, false>), grid, block, 0, s, y, slot_of, w, out, p.K, p.H);
  } else {
    const uint16_t* y = ws_at<uint16_t>(ws, p.off_y);
    if (out_bf16)
      BEAM_LAUNCH(tm, "combine", (combine<uint16_t, true>), grid, block, 0, s, y, slot_of, w, out, p.K, p.H);
    else
      BEAM_LAUNCH(tm, "combine", (combine<uint16_t, false>), grid, block, 0, s, y, slot_of, w, out, p.K, p.H);
  }
  return hipGetLastError();
}

}  // namespace beam
