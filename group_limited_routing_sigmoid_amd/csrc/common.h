// Device helpers shared by the gfx950 kernels of the Beam MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  bf16 b = static_cast<bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global load through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Buffer resource for raw 16-byte loads from base (bytes: the extent the
// hardware checks; loads past it return zeros).  Third word as gfx9 raw
// buffers take it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16-byte load at byte offset voff + soff from a buffer resource (soff
// wave-uniform: it goes in a scalar register).
__device__ __forceinline__ u32x4 buf16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds + 16*l, where lds must be the same for the
// whole wave.  Completion is tracked by the wave's vector-memory counter.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// As dma16 with 4 bytes per lane (lane l's dword lands at lds + 4*l).
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// D = A(32x16) * B(16x32) + C on the matrix cores, bf16 inputs, fp32 sums.
// Lane l supplies A row (l % 32) and B column (l % 32), k-block (l / 32).
// Accumulator element r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l supplies A row (l % 16) and B column
// (l % 16), k-block (l / 16).  Element r of lane l is C[4*(l/16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Four binary32 values -> four e4m3fn codes (byte j = value j) with the
// matrix-core conversion instruction: round to nearest even, sign kept, zero
// and subnormal codes as the format defines them.  It agrees with exact RNE
// for every |v| < 464 (checked on gfx950 over all code values, all midpoints
// and their neighbouring floats); from 464 up it gives the NaN code instead
// of saturating, so the values are first clamped to [-448, 448]: a block
// scale amax/448 rounded coarsely (a subnormal amax) can put v/scale past
// 448, and the recipe saturates such values.
__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true));
}

// silu(g) = g * sigmoid(g), the sigmoid from the hardware exponential and
// reciprocal (each within about 1 ulp of binary32).  The bf16 paths round
// silu(g) * u to 8 bits next, so an IEEE divide (about ten instructions more
// per output, most of a 256-row tile's epilogue) buys nothing there.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

}  // namespace beam
