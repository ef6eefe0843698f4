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

bool fp8_experts_built() { return false; }

hipError_t launch_experts_fp8(const Plan&, const void*, const uint8_t*,
                              const float*, const uint8_t*, const float*,
                              void*, hipStream_t, Timer*) {
  return hipErrorNotSupported;
}

}  // namespace beam
