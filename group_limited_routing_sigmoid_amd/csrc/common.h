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

__device__ __forceinline__ float silu(float g) {
  return g / (1.0f + __expf(-g));
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

}  // namespace beam
