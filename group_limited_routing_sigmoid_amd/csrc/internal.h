// Host-side plan of one call (shape, path choice, workspace carve-up) and the
// kernel launchers each translation unit provides.  Library-internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "beam_moe.h"

namespace beam {

// Grouped-GEMM row tile: rows (slots) per M tile of one expert (the bf16
// kernels also have 128- and 160-row forms, the MXFP4 kernels a 128-row form).
constexpr int kGemmBM = 256;
// Tokens routed per workgroup by the permutation kernels.
constexpr int kPermBlock = 256;

struct Plan {
  int32_t H, I, E, G, TG, K, topn;
  float scale;
  int32_t act, wdt;
  uint32_t flags;
  int64_t T, S;        // tokens, slots (= T*K)
  int64_t nb;          // permutation blocks
  int32_t ks;          // partial logits the router selection sums
  bool router_gemm;    // logits by the dense tile GEMM (many tokens)
  bool stream_path;    // weight-streaming experts (few tokens per expert)
  int32_t bm;          // rows per grouped-GEMM M tile: 256, 160 (bf16), 128 (bf16, MXFP4)
  int32_t xt;          // extra rows an expert's last M tile may hold (FP8: 32)
  int64_t max_tiles;   // upper bound on grouped-GEMM M tiles
  // byte offsets into the workspace
  size_t off_part, off_idx, off_w, off_hist, off_base, off_rank, off_counts,
      off_offsets, off_slot_token, off_slot_of,
      off_meta, off_active, off_tile_off, off_w3, off_h, off_y, off_xq, off_xs,
      off_hq, off_hs, off_xss;
  size_t total;
};

// Per-kernel event records for beam_moe_forward_timed (null: no timing).
struct Timer;
void timer_begin(Timer* t, const char* name, hipStream_t s);
void timer_end(Timer* t, hipStream_t s);

// Launch one kernel, bracketed by timer records when a timer is given.
#define BEAM_LAUNCH(tm, name, kernel, grid, block, shmem, stream, ...)   \
  do {                                                                    \
    timer_begin(tm, name, stream);                                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);  \
    timer_end(tm, stream);                                                \
  } while (0)

// Builds the plan; returns a beam_status.
int make_plan(const beam_moe_desc* d, int64_t T, Plan* p);

template <typename P>
static inline P* ws_at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// meta words (int32) at off_meta: [0] = grouped M tiles, [1] = active
// experts, [2] = M tiles of hot experts
constexpr int kMetaTiles = 0, kMetaActive = 1, kMetaHot = 2, kMetaWords = 4;

// An expert whose tokens fill at least this many M tiles reuses its weights
// over several tiles ("hot"); the others stream theirs once ("cold").
constexpr int kHotTiles = 2;

// Tile table (int32 words at off_tile_off), written by the permutation:
//   [0, E]            first M tile of each expert in the combined order: the
//                     hot experts' tiles first, then the cold experts', each
//                     group in expert order
//   [E + 1, 2E + 1)   M tiles of each expert
//   [2E + 2, ...)     the expert of each M tile of the combined order
__host__ __device__ constexpr int tt_count(int E) { return E + 1; }
__host__ __device__ constexpr int tt_expert(int E) { return 2 * E + 2; }

// router.hip
hipError_t launch_router(const Plan& p, const void* x, const float* w_router,
                         const float* bias, float* logits_out,
                         const float* logits_in, int32_t* idx, float* w,
                         void* ws, hipStream_t s, Timer* tm);
// experts_grouped.hip: router logits partials by the dense tile GEMM
hipError_t launch_router_gemm(const Plan& p, const void* x, const uint16_t* w3,
                              float* part, hipStream_t s, Timer* tm);
// permute.hip
hipError_t launch_permute(const Plan& p, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* slot_token,
                          int32_t* slot_of, void* ws, hipStream_t s, Timer* tm);
// mxfp4.hip (4-bit MX weights, MXFP8 activations)
hipError_t launch_quant_mxfp8(int64_t rows, int64_t cols, int32_t dtype, const void* v,
                              uint8_t* q, uint8_t* scales, hipStream_t s, Timer* tm);
hipError_t launch_experts_mxfp4(const Plan& p, const void* x, const uint8_t* w_gate_up,
                                const uint8_t* s_gate_up, const uint8_t* w_down,
                                const uint8_t* s_down, void* ws, hipStream_t s, Timer* tm);
hipError_t launch_bias_update(const Plan& p, const int32_t* idx, float gamma,
                              float* bias, hipStream_t s, Timer* tm);
// experts_grouped.hip (bf16 weights, tiled MFMA grouped GEMM)
hipError_t launch_grouped_bf16(const Plan& p, const void* x,
                               const void* w_gate_up, const void* w_down,
                               void* ws, hipStream_t s, Timer* tm);
// experts_stream.hip (bf16 weights, weight streaming)
hipError_t launch_stream_bf16(const Plan& p, const void* x,
                              const void* w_gate_up, const void* w_down,
                              void* ws, hipStream_t s, Timer* tm);
// experts_f32.hip (fp32 activations and weights)
hipError_t launch_experts_f32(const Plan& p, const float* x,
                              const float* w_gate_up, const float* w_down,
                              void* ws, hipStream_t s, Timer* tm);
// combine.hip
// Post-block epilogue fused into the combine: residual = a * residual +
// b * RMSNorm(block output) * gamma per token (a = sqrt((k-1)/k), b = 1/sqrt(k)).
struct Epilogue {
  const float* gamma;  // [H]
  float eps, a, b;
  float* residual;     // [T, H] fp32, in place
};

// out may be null when ep is given (the block output is then not stored).
hipError_t launch_combine(const Plan& p, const int32_t* slot_of,
                          const float* w, void* out, void* ws, hipStream_t s,
                          Timer* tm, const Epilogue* ep = nullptr);
// fp8.hip
hipError_t launch_quant_e4m3(int64_t rows, int64_t cols, int32_t dtype,
                             const void* v, uint8_t* q, float* scales,
                             hipStream_t s, Timer* tm);
bool fp8_experts_built();
hipError_t launch_experts_fp8(const Plan& p, const void* x,
                              const uint8_t* w_gate_up, const float* s_gate_up,
                              const uint8_t* w_down, const float* s_down,
                              void* ws, hipStream_t s, Timer* tm);

}  // namespace beam
