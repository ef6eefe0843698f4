// Expert MLPs in fp32 for fp32 activations and weights (small layers; one
// thread per output element, sequential fp32 fused multiply-adds).  Same
// SwiGLU expert as the bf16 paths ("Hugging Face releases Beam ..." MoE
// paragraph): h = silu(x W_g^T) * (x W_u^T), y = h W_d^T.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

// Expert of a slot: the e with offsets[e] <= slot < offsets[e+1].
__device__ __forceinline__ int slot_expert(const int32_t* offsets, int E, int slot) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (offsets[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void f32_gate_up(
    const float* __restrict__ x, const float* __restrict__ w_gu,
    float* __restrict__ h, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ offsets, int64_t S, int E, int H, int I) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= S * I) return;
  const int slot = static_cast<int>(i / I), c = static_cast<int>(i % I);
  const int e = slot_expert(offsets, E, slot);
  const float* xr = x + static_cast<int64_t>(slot_token[slot]) * H;
  const float* g = w_gu + (static_cast<int64_t>(e) * 2 * I + c) * H;
  const float* u = g + static_cast<int64_t>(I) * H;
  float ag = 0.0f, au = 0.0f;
  for (int k = 0; k < H; ++k) {
    ag = __builtin_fmaf(xr[k], g[k], ag);
    au = __builtin_fmaf(xr[k], u[k], au);
  }
  h[i] = silu(ag) * au;
}

__global__ __launch_bounds__(256) void f32_down(
    const float* __restrict__ h, const float* __restrict__ w_d,
    float* __restrict__ y, const int32_t* __restrict__ offsets, int64_t S,
    int E, int H, int I) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= S * H) return;
  const int slot = static_cast<int>(i / H), n = static_cast<int>(i % H);
  const int e = slot_expert(offsets, E, slot);
  const float* hr = h + static_cast<int64_t>(slot) * I;
  const float* wr = w_d + (static_cast<int64_t>(e) * H + n) * I;
  float a = 0.0f;
  for (int k = 0; k < I; ++k) a = __builtin_fmaf(hr[k], wr[k], a);
  y[i] = a;
}

}  // namespace

hipError_t launch_experts_f32(const Plan& p, const float* x,
                              const float* w_gate_up, const float* w_down,
                              void* ws, hipStream_t s, Timer* tm) {
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  float* h = ws_at<float>(ws, p.off_h);
  float* y = ws_at<float>(ws, p.off_y);
  BEAM_LAUNCH(tm, "f32_gate_up", f32_gate_up, dim3(static_cast<unsigned>(ceil_div(p.S * p.I, 256))),
                     dim3(256), 0, s, x, w_gate_up, h, slot_token, offsets, p.S,
                     p.E, p.H, p.I);
  BEAM_LAUNCH(tm, "f32_down", f32_down, dim3(static_cast<unsigned>(ceil_div(p.S * p.H, 256))),
                     dim3(256), 0, s, h, w_down, y, offsets, p.S, p.E, p.H, p.I);
  return hipGetLastError();
}

}  // namespace beam
