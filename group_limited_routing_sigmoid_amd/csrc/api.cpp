// C ABI of the Beam MoE block library: host-side validation, workspace plan,
// path choice and kernel launch order.  See include/beam_moe.h for the
// contract of every entry point.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "internal.h"

namespace beam {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? BEAM_OK : BEAM_ERR_HIP; }

}  // namespace

struct Timer {
  int32_t capacity = 0, count = 0;
  bool open = false;         // a begin without its end yet
  hipEvent_t* ev = nullptr;  // 2 * capacity events: start, stop pairs
  const char** names = nullptr;
};

void timer_begin(Timer* t, const char* name, hipStream_t s) {
  if (!t || t->count >= t->capacity) return;
  t->names[t->count] = name;
  hipEventRecord(t->ev[2 * t->count], s);
  t->open = true;
}

void timer_end(Timer* t, hipStream_t s) {
  if (!t || !t->open) return;
  hipEventRecord(t->ev[2 * t->count + 1], s);
  t->open = false;
  ++t->count;
}

int make_plan(const beam_moe_desc* d, int64_t T, Plan* p) {
  const int st = beam_moe_validate(d, T);
  if (st != BEAM_OK) return st;
  memset(p, 0, sizeof(*p));
  p->H = d->hidden;
  p->I = d->intermediate;
  p->E = d->n_experts;
  p->G = d->n_groups;
  p->TG = d->topk_groups;
  p->K = d->top_k;
  p->topn = d->group_score_topn;
  p->scale = d->routed_scale;
  p->act = d->act_dtype;
  p->wdt = d->weight_dtype;
  p->flags = d->flags;
  p->T = T;
  p->S = T * d->top_k;
  p->nb = ceil_div(T, kPermBlock);
  // Router reduction split: enough waves to spread W_r over the chip when
  // there are few tokens; each split must cover a multiple of 16 columns.
  p->ks = 1;
  p->router_gemm = p->act == BEAM_BF16 && p->E % 256 == 0 && T >= 1024;
  if (p->router_gemm) {
    // dense tile GEMM of x against W3 = the three bf16 terms of W_r side by
    // side (depth 3H); split the depth until about one workgroup per
    // compute unit
    const int64_t tiles = ceil_div(T, kGemmBM) * (p->E / 256);
    p->ks = 1;
    while (p->ks < 16 && tiles * p->ks < 256 && (3 * p->H / 64) % (2 * p->ks) == 0)
      p->ks *= 2;
  } else if (p->act == BEAM_BF16 && p->E % 32 == 0) {
    // four waves per workgroup, each taking a quarter of the split's columns
    const int64_t waves = ceil_div(T, 32) * ceil_div(p->E, 64) * 4;
    while (p->ks < 16 && waves * p->ks < 2048 && (p->H / 16) % (8 * p->ks) == 0)
      p->ks *= 2;
  }
  // Very few tokens per expert: stream each touched expert's weights once.
  // Measured on the Beam layer, bf16: streaming 0.34 / 0.54 / 0.82 ms vs
  // 128-row grouped tiles 0.39 / 0.57 / 0.87 ms at T = 2 / 4 / 8, grouped
  // ahead from T = 16 (1.40 vs 1.43 ms) on; so streaming while T*K < E/2.
  if (p->flags & BEAM_PATH_STREAM)
    p->stream_path = true;
  else if (p->flags & BEAM_PATH_GROUPED)
    p->stream_path = false;
  else
    p->stream_path = 2 * p->S < static_cast<int64_t>(p->E);
  // streaming kernels exist for bf16 weights only
  if (p->wdt != BEAM_BF16) p->stream_path = false;
  // 4-bit MX weights: the grouped tiles with their copy rings are ahead at
  // every batch measured (T = 1: 0.189 vs 0.215 ms streaming, T = 8: 0.437
  // vs 0.500, T = 64: 1.25 vs 1.60); the streaming kernels run when asked for
  if (p->wdt == BEAM_MXFP4) p->stream_path = (p->flags & BEAM_PATH_STREAM) != 0;
  const int64_t S = p->S, E = p->E, H = p->H, I = p->I;
  // Grouped tiles of 128 (or, bf16, 160) rows with a deeper copy ring while
  // the experts hold few rows, 256 rows above; measured on the Beam layer.
  // bf16, 128 / 256 rows (the four-wave 256-row tiles with triple-buffered
  // weights): 3.77 / 3.82 ms at 2K tokens, 3.88 / 3.93 at 2.5K, 4.16 / 4.02
  // at 3K, and 256 rows 4.19 ms at 4K against 4.72 for the 160-row ring; so
  // 128 below T*K = 96E, 256 above (160 rows on request).  MXFP4, 128 / 256 rows: 1.57 /
  // 1.61 ms at 1K tokens, 2.77 / 2.38 at 4K; so 128 below T*K = 32E.  FP8,
  // 128 / 256 (+32) rows: 1.63 / 1.99 ms at 64 tokens, 2.28 / 2.60 at 2K,
  // 2.76 / 2.93 at 3.5K, 3.31 / 3.02 at 4K; so 128 below T*K = 120E.
  p->bm = kGemmBM;
  if (p->wdt == BEAM_BF16) {
    if (p->flags & (BEAM_TILE_64 | BEAM_TILE_128)) p->bm = 128;
    else if (p->flags & BEAM_TILE_160) p->bm = 160;
    else if (p->flags & BEAM_TILE_256) p->bm = kGemmBM;
    else if (S < 96 * E) p->bm = 128;
  } else if (p->wdt == BEAM_MXFP4) {
    // 64-slot tiles with 256-deep stages (H, I multiples of 512) against the
    // rest at default: 1.02 / 1.11 ms at 64 tokens, 1.33 / 1.46 at 1K, 1.44
    // / 1.55 at 1.5K, 1.71 / 1.68 at 2K, 2.21 / 1.91 at 3K
    const bool wide = H % 512 == 0 && I % 512 == 0;
    if (p->flags & BEAM_TILE_64) p->bm = 64;
    else if (p->flags & BEAM_TILE_128) p->bm = 128;
    else if (p->flags & (BEAM_TILE_160 | BEAM_TILE_256)) p->bm = kGemmBM;
    else if (wide && S < 56 * E) p->bm = 64;
    else if (S < 32 * E) p->bm = 128;
  } else if (p->wdt == BEAM_FP8_E4M3) {
    if (p->flags & (BEAM_TILE_64 | BEAM_TILE_128)) p->bm = 128;
    else if (!(p->flags & (BEAM_TILE_160 | BEAM_TILE_256)) && S < 120 * E) p->bm = 128;
  }
  // FP8, and MXFP4 where its 256-slot tiles run two stages (T*K >= 192E):
  // an expert's last tile takes up to 32 rows past 256, so experts near 256
  // rows need one tile, not a full one plus a sliver
  p->xt = 0;
  if (!(p->flags & BEAM_TILE_256) && p->bm == kGemmBM) {
    if (p->wdt == BEAM_FP8_E4M3) p->xt = 32;
    if (p->wdt == BEAM_MXFP4 && S >= 192 * E) p->xt = 32;
  }
  p->max_tiles = S / p->bm + (S < E ? S : E) + 1;
  const bool f32 = p->wdt == BEAM_F32;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  p->off_part = take(static_cast<size_t>(p->ks) * T * E * 4);
  p->off_w3 = p->router_gemm ? take(3 * E * H * 2) : 0;
  p->off_idx = take(S * 4);
  p->off_w = take(S * 4);
  p->off_hist = take(p->nb * E * 4);
  p->off_base = take(p->nb * E * 4);
  p->off_rank = take(S * 4);
  p->off_counts = take(E * 4);
  p->off_offsets = take((E + 1) * 4);
  p->off_slot_token = take(S * 4);
  p->off_slot_of = take(S * 4);
  p->off_meta = take(kMetaWords * 4);
  p->off_active = take(E * 4);
  p->off_tile_off = take((tt_expert(static_cast<int>(E)) + p->max_tiles) * 4);
  // h is fp32 on the fp32 path and before the MXFP8 quantisation of the
  // streaming 4-bit path, bf16 otherwise; the grouped e4m3 and 4-bit gate/up
  // GEMMs write only its codes
  const bool h_codes_only = p->wdt == BEAM_FP8_E4M3 || (p->wdt == BEAM_MXFP4 && !p->stream_path);
  p->off_h = take(h_codes_only ? 0 : S * I * ((f32 || p->wdt == BEAM_MXFP4) ? 4 : 2));
  p->off_y = take(S * H * ((f32 || p->stream_path || p->wdt == BEAM_MXFP4) ? 4 : 2));
  if (p->wdt == BEAM_MXFP4) {
    // grouped path: x's E8M0 bytes also per slot, as one word per 128 k,
    // block-major ([H/128][S] words), and h's the same ([I/128][S])
    p->off_xq = take(T * H);
    p->off_xs = take(T * (H / 32));
    p->off_xss = p->stream_path ? 0 : take(S * (H / 32));
    p->off_hq = take(S * I);
    p->off_hs = take(S * (I / 32));
  }
  if (p->wdt == BEAM_FP8_E4M3) {
    // x's scales per token, then per slot and block-major ([H/128][S]), as
    // are h's ([I/128][S]): a tile stage reads the words of consecutive slots
    p->off_xq = take(T * H);
    p->off_xs = take(T * (H / 128) * 4);
    p->off_xss = take(S * (H / 128) * 4);
    p->off_hq = take(S * I);
    p->off_hs = take(S * (I / 128) * 4);
  }
  p->total = o;
  return BEAM_OK;
}

}  // namespace beam

using namespace beam;

extern "C" {

const char* beam_status_string(int status) {
  switch (status) {
    case BEAM_OK: return "ok";
    case BEAM_ERR_INVALID_ARG: return "invalid argument";
    case BEAM_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BEAM_ERR_WORKSPACE: return "workspace missing or too small";
    case BEAM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int beam_moe_validate(const beam_moe_desc* d, int64_t T) {
  if (!d || T < 0) return BEAM_ERR_INVALID_ARG;
  const uint32_t tiles = BEAM_TILE_64 | BEAM_TILE_128 | BEAM_TILE_160 | BEAM_TILE_256;
  const uint32_t known = BEAM_ROUTE_LOGITS_IN | BEAM_PATH_STREAM | BEAM_PATH_GROUPED | tiles;
  if (d->flags & ~known) return BEAM_ERR_INVALID_ARG;
  const uint32_t tf = d->flags & tiles;
  if (tf & (tf - 1)) return BEAM_ERR_INVALID_ARG;  // at most one tile height
  if ((d->flags & BEAM_PATH_STREAM) && (d->flags & BEAM_PATH_GROUPED))
    return BEAM_ERR_INVALID_ARG;
  if (d->act_dtype != BEAM_F32 && d->act_dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
  if (d->weight_dtype != BEAM_F32 && d->weight_dtype != BEAM_BF16 &&
      d->weight_dtype != BEAM_FP8_E4M3 && d->weight_dtype != BEAM_MXFP4)
    return BEAM_ERR_INVALID_ARG;
  if (!(d->routed_scale > 0.0f) || !isfinite(d->routed_scale)) return BEAM_ERR_INVALID_ARG;
  const int E = d->n_experts, G = d->n_groups;
  if (E < 1 || E > 1024 || G < 1 || G > 64 || E % G) return BEAM_ERR_UNSUPPORTED;
  const int gs = E / G;
  if (gs > 64) return BEAM_ERR_UNSUPPORTED;
  if (d->topk_groups < 1 || d->topk_groups > G) return BEAM_ERR_UNSUPPORTED;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->topk_groups * gs)
    return BEAM_ERR_UNSUPPORTED;
  if (d->group_score_topn < 1 || d->group_score_topn > 2 || d->group_score_topn > gs)
    return BEAM_ERR_UNSUPPORTED;
  if (d->hidden < 128 || d->hidden % 128 || d->intermediate < 128 ||
      d->intermediate % 128)
    return BEAM_ERR_UNSUPPORTED;
  if (d->weight_dtype == BEAM_F32 && d->act_dtype != BEAM_F32) return BEAM_ERR_UNSUPPORTED;
  if (d->weight_dtype != BEAM_F32 && d->act_dtype != BEAM_BF16) return BEAM_ERR_UNSUPPORTED;
  // slot indices and per-slot element offsets are 32-bit
  const int64_t S = T * static_cast<int64_t>(d->top_k);
  const int64_t wide = d->hidden > d->intermediate ? d->hidden : d->intermediate;
  if (S * wide > 0x7FFFFFFF) return BEAM_ERR_UNSUPPORTED;
  // element (bf16, fp32) and byte (e4m3, 4-bit) offsets inside one expert's
  // weights are 32-bit: its gate/up matrix holds 2*I*H values
  if (2 * static_cast<int64_t>(d->intermediate) * d->hidden > 0x7FFFFFFF)
    return BEAM_ERR_UNSUPPORTED;
  return BEAM_OK;
}

int beam_moe_workspace_bytes(const beam_moe_desc* d, int64_t T, size_t* bytes) {
  if (!bytes) return BEAM_ERR_INVALID_ARG;
  Plan p;
  const int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  *bytes = T == 0 ? 0 : p.total;
  return BEAM_OK;
}

int beam_moe_route(const beam_moe_desc* d, int64_t T, const void* x,
                   const float* w_router, const float* bias, float* logits,
                   int32_t* topk_idx, float* topk_w, void* workspace,
                   size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  const bool lin = d->flags & BEAM_ROUTE_LOGITS_IN;
  if (!topk_idx || !topk_w) return BEAM_ERR_INVALID_ARG;
  if (lin ? !logits : (!x || !w_router)) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(bias) ||
      !aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w))
    return BEAM_ERR_INVALID_ARG;
  if (!lin) {
    if (!workspace || ws_bytes < p.total) return BEAM_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return BEAM_ERR_INVALID_ARG;
  }
  return hip_status(launch_router(p, x, w_router, bias, lin ? nullptr : logits,
                                  lin ? logits : nullptr, topk_idx, topk_w,
                                  workspace, static_cast<hipStream_t>(stream),
                                  nullptr));
}

int beam_moe_permute(const beam_moe_desc* d, int64_t T, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* slot_token,
                     int32_t* slot_of, void* workspace, size_t ws_bytes,
                     void* stream) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  if (!topk_idx || !counts || !offsets || !slot_token || !slot_of)
    return BEAM_ERR_INVALID_ARG;
  if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) ||
      !aligned16(slot_token) || !aligned16(slot_of))
    return BEAM_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < p.total) return BEAM_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return BEAM_ERR_INVALID_ARG;
  return hip_status(launch_permute(p, topk_idx, counts, offsets, slot_token,
                                   slot_of, workspace, static_cast<hipStream_t>(stream),
                                   nullptr));
}

int beam_moe_bias_update(const beam_moe_desc* d, int64_t T, const int32_t* topk_idx,
                         float gamma, float* bias, void* stream) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (!(gamma >= 0.0f) || !isfinite(gamma)) return BEAM_ERR_INVALID_ARG;
  if (T == 0) return BEAM_OK;
  if (!topk_idx || !bias || !aligned16(topk_idx) || !aligned16(bias))
    return BEAM_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(p, topk_idx, gamma, bias,
                                       static_cast<hipStream_t>(stream), nullptr));
}

float beam_moe_bias_gamma(int64_t t, int64_t n, float g0, float g1) {
  if (n <= 0) return g1;
  if (t < 0) t = 0;
  if (t > n) t = n;
  const double c = 0.5 * (1.0 + cos(M_PI * static_cast<double>(t) / static_cast<double>(n)));
  return static_cast<float>(static_cast<double>(g1) + (static_cast<double>(g0) - g1) * c);
}

int beam_moe_quant_e4m3(int64_t rows, int64_t cols, int32_t dtype,
                        const void* v, uint8_t* q, float* scales, void* stream) {
  if (rows < 0 || cols < 0 || (dtype != BEAM_F32 && dtype != BEAM_BF16))
    return BEAM_ERR_INVALID_ARG;
  if (cols % 128) return BEAM_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return BEAM_OK;
  if (!v || !q || !scales || !aligned16(v) || !aligned16(q) || !aligned16(scales))
    return BEAM_ERR_INVALID_ARG;
  return hip_status(launch_quant_e4m3(rows, cols, dtype, v, q, scales,
                                      static_cast<hipStream_t>(stream), nullptr));
}

int beam_moe_quant_mxfp8(int64_t rows, int64_t cols, int32_t dtype,
                         const void* v, uint8_t* q, uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || (dtype != BEAM_F32 && dtype != BEAM_BF16))
    return BEAM_ERR_INVALID_ARG;
  if (cols % 128) return BEAM_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return BEAM_OK;
  if (!v || !q || !scales || !aligned16(v) || !aligned16(q) || !aligned16(scales))
    return BEAM_ERR_INVALID_ARG;
  return hip_status(launch_quant_mxfp8(rows, cols, dtype, v, q, scales,
                                       static_cast<hipStream_t>(stream), nullptr));
}

static int forward_impl(const beam_moe_desc* d, int64_t T, const void* x,
                        const float* w_router, const float* bias,
                        const void* w_gate_up, const void* s_gate_up,
                        const void* w_down, const void* s_down, void* out,
                        int32_t* topk_idx, float* topk_w, float* logits,
                        void* workspace, size_t ws_bytes, void* stream,
                        Timer* tm, const Epilogue* ep = nullptr) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  const bool lin = d->flags & BEAM_ROUTE_LOGITS_IN;
  const bool fp8 = d->weight_dtype == BEAM_FP8_E4M3;
  const bool mx4 = d->weight_dtype == BEAM_MXFP4;
  if (!x || !w_gate_up || !w_down || (!out && !ep)) return BEAM_ERR_INVALID_ARG;
  if (lin ? !logits : !w_router) return BEAM_ERR_INVALID_ARG;
  if ((fp8 || mx4) && (!s_gate_up || !s_down)) return BEAM_ERR_INVALID_ARG;
  if (fp8 && !fp8_experts_built()) return BEAM_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, w_router, bias, w_gate_up, s_gate_up, w_down,
                        s_down, out, topk_idx, topk_w, logits};
  for (const void* q : ptrs)
    if (!aligned16(q)) return BEAM_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < p.total) return BEAM_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return BEAM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : ws_at<int32_t>(workspace, p.off_idx);
  float* w = topk_w ? topk_w : ws_at<float>(workspace, p.off_w);
  hipError_t e = launch_router(p, x, w_router, bias, lin ? nullptr : logits,
                               lin ? logits : nullptr, idx, w, workspace, s, tm);
  if (e != hipSuccess) return BEAM_ERR_HIP;
  int32_t* slot_of = ws_at<int32_t>(workspace, p.off_slot_of);
  e = launch_permute(p, idx, ws_at<int32_t>(workspace, p.off_counts),
                     ws_at<int32_t>(workspace, p.off_offsets),
                     ws_at<int32_t>(workspace, p.off_slot_token), slot_of,
                     workspace, s, tm);
  if (e != hipSuccess) return BEAM_ERR_HIP;
  if (p.wdt == BEAM_F32)
    e = launch_experts_f32(p, static_cast<const float*>(x),
                           static_cast<const float*>(w_gate_up),
                           static_cast<const float*>(w_down), workspace, s, tm);
  else if (fp8)
    e = launch_experts_fp8(p, x, static_cast<const uint8_t*>(w_gate_up),
                           static_cast<const float*>(s_gate_up),
                           static_cast<const uint8_t*>(w_down),
                           static_cast<const float*>(s_down), workspace, s, tm);
  else if (mx4)
    e = launch_experts_mxfp4(p, x, static_cast<const uint8_t*>(w_gate_up),
                             static_cast<const uint8_t*>(s_gate_up),
                             static_cast<const uint8_t*>(w_down),
                             static_cast<const uint8_t*>(s_down), workspace, s, tm);
  else if (p.stream_path)
    e = launch_stream_bf16(p, x, w_gate_up, w_down, workspace, s, tm);
  else
    e = launch_grouped_bf16(p, x, w_gate_up, w_down, workspace, s, tm);
  if (e != hipSuccess) return BEAM_ERR_HIP;
  return hip_status(launch_combine(p, slot_of, w, out, workspace, s, tm, ep));
}

int beam_moe_forward(const beam_moe_desc* d, int64_t T, const void* x,
                     const float* w_router, const float* bias,
                     const void* w_gate_up, const void* s_gate_up,
                     const void* w_down, const void* s_down, void* out,
                     int32_t* topk_idx, float* topk_w, float* logits,
                     void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(d, T, x, w_router, bias, w_gate_up, s_gate_up, w_down,
                      s_down, out, topk_idx, topk_w, logits, workspace,
                      ws_bytes, stream, nullptr);
}

int beam_moe_forward_residual(const beam_moe_desc* d, int64_t T, const void* x,
                              const float* w_router, const float* bias,
                              const void* w_gate_up, const void* s_gate_up,
                              const void* w_down, const void* s_down,
                              const float* norm_weight, float eps, int32_t step,
                              float* residual, void* out, void* workspace,
                              size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (step < 1 || !(eps >= 0.0f) || !isfinite(eps)) return BEAM_ERR_INVALID_ARG;
  // the token's fp32 row is held in dynamic LDS between the norm's two
  // passes; 64 KiB is the dynamic size every launch gets without attributes
  if (static_cast<int64_t>(d->hidden) * 4 > 64 * 1024) return BEAM_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_OK;
  if (!norm_weight || !residual || !aligned16(norm_weight) || !aligned16(residual))
    return BEAM_ERR_INVALID_ARG;
  Epilogue ep;
  ep.gamma = norm_weight;
  ep.eps = eps;
  ep.a = static_cast<float>(sqrt(static_cast<double>(step - 1) / static_cast<double>(step)));
  ep.b = static_cast<float>(1.0 / sqrt(static_cast<double>(step)));
  ep.residual = residual;
  return forward_impl(d, T, x, w_router, bias, w_gate_up, s_gate_up, w_down, s_down, out,
                      nullptr, nullptr, nullptr, workspace, ws_bytes, stream, nullptr, &ep);
}

}  // extern "C"

// ---- forward for callers that cannot allocate ------------------------------
// The workspace of beam_moe_forward_noalloc: a file-scope device array; every
// GPU the library runs on holds its own copy until the process ends.  In
// host code its name is a host-side stand-in, not a device address: host
// code uses only the per-device address looked up below.
static __device__ __align__(256) unsigned char scratch[BEAM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Address of the current device's copy of `scratch`, looked up once per
// device with that device current.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BEAM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BEAM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BEAM_OK;
}

}  // namespace

extern "C" {

int beam_moe_forward_noalloc(const beam_moe_desc* d, int64_t T, const void* x,
                             const float* w_router, const float* bias,
                             const void* w_gate_up, const void* s_gate_up,
                             const void* w_down, const void* s_down, void* out,
                             int32_t* topk_idx, float* topk_w, float* logits,
                             void* stream) {
  Plan p;
  int st = make_plan(d, T, &p);
  if (st != BEAM_OK) return st;
  if (T == 0) return BEAM_OK;
  if (p.total > BEAM_NOALLOC_SCRATCH_BYTES) return BEAM_ERR_WORKSPACE;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != BEAM_OK) return st;
  return forward_impl(d, T, x, w_router, bias, w_gate_up, s_gate_up, w_down, s_down,
                      out, topk_idx, topk_w, logits, ws, BEAM_NOALLOC_SCRATCH_BYTES,
                      stream, nullptr);
}

int beam_moe_forward_timed(const beam_moe_desc* d, int64_t T, const void* x,
                           const float* w_router, const float* bias,
                           const void* w_gate_up, const void* s_gate_up,
                           const void* w_down, const void* s_down, void* out,
                           int32_t* topk_idx, float* topk_w, float* logits,
                           void* workspace, size_t ws_bytes, void* stream,
                           beam_moe_timer* timer) {
  return forward_impl(d, T, x, w_router, bias, w_gate_up, s_gate_up, w_down,
                      s_down, out, topk_idx, topk_w, logits, workspace,
                      ws_bytes, stream, reinterpret_cast<Timer*>(timer));
}

int beam_moe_timer_create(int32_t capacity, beam_moe_timer** out) {
  if (!out) return BEAM_ERR_INVALID_ARG;
  *out = nullptr;
  if (capacity < 1) return BEAM_ERR_INVALID_ARG;
  Timer* t = new Timer;
  t->capacity = capacity;
  t->ev = new hipEvent_t[2 * static_cast<size_t>(capacity)]();
  t->names = new const char*[capacity]();
  for (int32_t i = 0; i < 2 * capacity; ++i)
    if (hipEventCreate(&t->ev[i]) != hipSuccess) {
      for (int32_t j = 0; j < i; ++j) hipEventDestroy(t->ev[j]);
      delete[] t->ev;
      delete[] t->names;
      delete t;
      return BEAM_ERR_HIP;
    }
  *out = reinterpret_cast<beam_moe_timer*>(t);
  return BEAM_OK;
}

void beam_moe_timer_destroy(beam_moe_timer* timer) {
  Timer* t = reinterpret_cast<Timer*>(timer);
  if (!t) return;
  for (int32_t i = 0; i < 2 * t->capacity; ++i) hipEventDestroy(t->ev[i]);
  delete[] t->ev;
  delete[] t->names;
  delete t;
}

void beam_moe_timer_reset(beam_moe_timer* timer) {
  Timer* t = reinterpret_cast<Timer*>(timer);
  if (t) {
    t->count = 0;
    t->open = false;
  }
}

int32_t beam_moe_timer_count(const beam_moe_timer* timer) {
  const Timer* t = reinterpret_cast<const Timer*>(timer);
  return t ? t->count : 0;
}

int beam_moe_timer_read(beam_moe_timer* timer, int32_t i, const char** name,
                        float* ms) {
  Timer* t = reinterpret_cast<Timer*>(timer);
  if (!t || i < 0 || i >= t->count || !name || !ms) return BEAM_ERR_INVALID_ARG;
  if (hipEventSynchronize(t->ev[2 * i + 1]) != hipSuccess) return BEAM_ERR_HIP;
  if (hipEventElapsedTime(ms, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess)
    return BEAM_ERR_HIP;
  *name = t->names[i];
  return BEAM_OK;
}

}  // extern "C"
