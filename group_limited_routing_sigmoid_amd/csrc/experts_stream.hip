// Expert MLPs for decode-sized batches: each touched expert sees only a few
// tokens, so the work is bound by reading its weights once from HBM.  The
// weights are the 16-row A side of 16x16x32 bf16 MFMA and up to 16 tokens
// are the B side.  Gate/up: one wave streams 16 rows (8 gate, 8 up) over
// the whole hidden dimension; down: one wave streams 16 rows of W_d over the
// whole intermediate dimension.  No cross-wave reduction.  Experts with more
// than 16 tokens are handled in chunks of 16.
//
// Same SwiGLU expert as the grouped path ("Hugging Face releases Beam ..."
// MoE paragraph): h = silu(x W_g^T) * (x W_u^T) for gate/up, y = h W_d^T for
// down.  h is kept in bf16 (the down product's input); y in fp32.
//
// Work items: (active expert j, 8-channel block) for gate/up and (active
// expert j, 16-row block of W_d) for down.  The grid covers every expert
// that could be active; items past the device-side count exit at once, so
// the host never waits for the routing result.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

// Gate/up: one wave per (active expert j, 8-channel block cb).  Its 16-row
// A side holds the gate rows of channels cb*8 .. +8 (rows 0..7) and the
// matching up rows (8..15), streamed over the whole hidden dimension with 20
// loads of 1 KiB in flight (the down kernel's shape); one accumulator covers
// both halves, and the up value of gate row g sits 32 lanes further (row
// 8 + g), fetched across lanes for silu(g)*u.
// grid ceil(max_active * I/8 / 4), block 256.
#ifndef BEAM_GU_UNROLL
#define BEAM_GU_UNROLL 20
#endif
constexpr int kGuUnroll = BEAM_GU_UNROLL;  // k-steps of 32 in flight per wave

__global__ __launch_bounds__(kThreads) void stream_gate_up(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_gu,
    uint16_t* __restrict__ h, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ meta,
    int H, int I) {
  const int n_cb = I / 8;
  const int item = blockIdx.x * kWaves + threadIdx.x / kWave;
  const int j = item / n_cb;
  const int cb = item % n_cb;
  if (j >= meta[kMetaActive]) return;
  const int e = active[j];
  const int off = offsets[e], cnt = counts[e];
  const int lane = threadIdx.x % kWave;
  const int row = lane % 16;
  const int kofs = 8 * (lane / 16);
  const int wrow = (row < 8) ? (cb * 8 + row) : (I + cb * 8 + (row - 8));
  const uint16_t* w0 = w_gu + (static_cast<int64_t>(e) * 2 * I + wrow) * H + kofs;
  for (int c0 = 0; c0 < cnt; c0 += 16) {
    const int ntok = min(16, cnt - c0);
    const bool has_tok = (lane % 16) < ntok;
    const uint16_t* xr = x + (has_tok ? static_cast<int64_t>(slot_token[off + c0 + lane % 16]) * H : 0) + kofs;
    f32x4 a0 = {}, a1 = {};
    for (int k = 0; k < H; k += 32 * kGuUnroll) {
      u32x4 wv[kGuUnroll], xb[kGuUnroll];
#pragma unroll
      for (int u = 0; u < kGuUnroll; ++u) {
        const bool in = k + 32 * u < H;
        wv[u] = in ? ld16(w0 + k + 32 * u) : u32x4{0, 0, 0, 0};
        xb[u] = (in && has_tok) ? ld16(xr + k + 32 * u) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kGuUnroll; ++u) {
        if (u % 2 == 0) a0 = mfma16x16x32(as_bf16x8(wv[u]), as_bf16x8(xb[u]), a0);
        else            a1 = mfma16x16x32(as_bf16x8(wv[u]), as_bf16x8(xb[u]), a1);
      }
    }
    const f32x4 g = a0 + a1;
    // element r of lane l: row 4*(l/16) + r, token l%16; lanes 0..31 hold the
    // gate rows 0..7, lanes 32..63 the up rows 8..15 of the same channels
    f32x4 u;
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = __shfl(g[r], (lane + 32) % kWave);
    if (lane < 32 && has_tok) {
      uint16_t* hr = h + static_cast<int64_t>(off + c0 + lane % 16) * I + cb * 8 + 4 * (lane / 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) hr[r] = f32_to_bf16_bits(silu(g[r]) * u[r]);
    }
  }
}

// Down: one wave per (active expert j, 16-row block of W_d), streaming the
// 16 rows over the whole intermediate dimension with two accumulator chains
// (even and odd k-steps) added once at the end.
// grid ceil(max_active * H/16 / 4), block 256 (4 work items per workgroup)
#ifndef BEAM_DN_UNROLL
#define BEAM_DN_UNROLL 20
#endif
constexpr int kDnUnroll = BEAM_DN_UNROLL;  // k-steps of 32 in flight per wave

__global__ __launch_bounds__(kThreads) void stream_down(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_d,
    float* __restrict__ y, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ meta, int H, int I) {
  const int n_ob = H / 16;
  const int item = blockIdx.x * kWaves + threadIdx.x / kWave;
  const int j = item / n_ob;
  const int ob = item % n_ob;
  if (j >= meta[kMetaActive]) return;
  const int e = active[j];
  const int off = offsets[e], cnt = counts[e];
  const int lane = threadIdx.x % kWave;
  const int kofs = 8 * (lane / 16);
  const uint16_t* w0 = w_d + (static_cast<int64_t>(e) * H + ob * 16 + lane % 16) * I + kofs;

  for (int c0 = 0; c0 < cnt; c0 += 16) {
    const int ntok = min(16, cnt - c0);
    const bool has_tok = (lane % 16) < ntok;
    const uint16_t* hr = h + static_cast<int64_t>(off + c0 + (has_tok ? lane % 16 : 0)) * I + kofs;
    f32x4 a0 = {}, a1 = {};
    for (int k = 0; k < I; k += 32 * kDnUnroll) {
      u32x4 wv[kDnUnroll], hb[kDnUnroll];
#pragma unroll
      for (int u = 0; u < kDnUnroll; ++u) {
        const bool in = k + 32 * u < I;
        wv[u] = in ? ld16(w0 + k + 32 * u) : u32x4{0, 0, 0, 0};
        hb[u] = (in && has_tok) ? ld16(hr + k + 32 * u) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kDnUnroll; ++u) {
        if (u % 2 == 0) a0 = mfma16x16x32(as_bf16x8(wv[u]), as_bf16x8(hb[u]), a0);
        else            a1 = mfma16x16x32(as_bf16x8(wv[u]), as_bf16x8(hb[u]), a1);
      }
    }
    const f32x4 r = a0 + a1;
    if (has_tok) {
      // element q: row ob*16 + 4*(lane/16) + q of W_d, token lane%16
      float* yr = y + static_cast<int64_t>(off + c0 + lane % 16) * H + ob * 16 + 4 * (lane / 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) yr[q] = r[q];
    }
  }
}

}  // namespace

hipError_t launch_stream_bf16(const Plan& p, const void* x,
                              const void* w_gate_up, const void* w_down,
                              void* ws, hipStream_t s, Timer* tm) {
  const int32_t* slot_token = ws_at<int32_t>(ws, p.off_slot_token);
  const int32_t* counts = ws_at<int32_t>(ws, p.off_counts);
  const int32_t* offsets = ws_at<int32_t>(ws, p.off_offsets);
  const int32_t* active = ws_at<int32_t>(ws, p.off_active);
  const int32_t* meta = ws_at<int32_t>(ws, p.off_meta);
  uint16_t* h = ws_at<uint16_t>(ws, p.off_h);
  float* y = ws_at<float>(ws, p.off_y);
  const int64_t max_active = p.S < p.E ? p.S : p.E;
  BEAM_LAUNCH(tm, "stream_gate_up_bf16", stream_gate_up,
              dim3(static_cast<unsigned>(ceil_div(max_active * (p.I / 8), kWaves))),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w_gate_up), h, slot_token,
                     counts, offsets, active, meta, p.H, p.I);
  BEAM_LAUNCH(tm, "stream_down_bf16", stream_down,
              dim3(static_cast<unsigned>(ceil_div(max_active * (p.H / 16), kWaves))),
                     dim3(kThreads), 0, s, h, static_cast<const uint16_t*>(w_down),
                     y, counts, offsets, active, meta, p.H, p.I);
  return hipGetLastError();
}

}  // namespace beam
