/*
 * beam_moe.h -- C ABI of the MI355X (gfx950) Beam MoE block library.
 *
 * One forward pass of the Mixture-of-Experts block of the Beam model:
 *   router    sigmoid scores over E experts in G contiguous groups, a
 *             per-expert bias that steers selection only, group score = sum
 *             of the group's best two biased scores, keep the best TG
 *             groups, pick the top K experts inside them, normalise the K
 *             unbiased scores to sum 1 and multiply by the routed scale;
 *   experts   K SwiGLU MLPs per token: h = silu(x W_g^T) * (x W_u^T),
 *             y = h W_d^T, no shared expert;
 *   combine   out = sum_k w_k y_k in rank order.
 * Sources: "Hugging Face releases Beam, a 501B-parameter open
 * Mixture-of-Experts model with 1M-token context" (MoE paragraph: 256
 * experts, SwiGLU intermediate 2,560, top 8 of the top 4 of 8 groups of 32);
 * "Reflection Releases Beam: An Open 501B-Parameter MoE Model Under Apache
 * 2.0", section "Where Beam Saves and Where the Memory Bill Comes In" (no
 * shared expert, DeepSeek-V3 group-limited sigmoid router, weights
 * normalised and scaled by 2.5); "Reflection AI Introduces Beam ..." (load
 * balancing by a DeepSeek-V3-style expert bias).  The group-score rule is
 * DeepSeek-V3's (arXiv 2412.19437, section 2.1.2); the pages invoke that
 * scheme without spelling the rule out.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller.  The
 *     library allocates nothing, frees nothing and keeps no pointer after a
 *     call returns.  Scratch memory is the caller's workspace, sized by
 *     beam_moe_workspace_bytes().
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream) and is asynchronous: the call returns once the
 *     kernels are launched.  Errors inside kernels surface at the caller's
 *     next synchronisation.
 *   - Argument, shape and workspace errors are detected on the host before
 *     anything is launched (no partial work) and returned as a negative
 *     beam_status.  No exceptions cross the ABI.  T == 0 is a no-op.
 *   - Device pointers must be 16-byte aligned; the workspace 256-byte aligned.
 *   - Layouts are row-major.  Weights use the out x in ("nn.Linear") layout.
 *   - Identical inputs give bitwise identical outputs (no floating-point
 *     atomics).  Calls are reentrant given distinct workspaces.
 *   - Inputs containing NaN or Inf are outside the contract.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BEAM_OK = 0,
  BEAM_ERR_INVALID_ARG = -1, /* null pointer, misalignment, T < 0, bad enum */
  BEAM_ERR_UNSUPPORTED = -2, /* a shape or dtype combination not built here */
  BEAM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  BEAM_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} beam_status;

typedef enum {
  BEAM_F32 = 0,      /* IEEE binary32 */
  BEAM_BF16 = 1,     /* bfloat16 */
  BEAM_FP8_E4M3 = 2, /* OCP e4m3fn codes with per-128x128-block fp32 scales */
  BEAM_MXFP4 = 3     /* OCP MX FP4: E2M1 codes two per byte (even k in the low
                        nibble), one E8M0 scale byte per 32 k of a row */
} beam_dtype;

/* flags */
#define BEAM_ROUTE_LOGITS_IN (1u << 0) /* route from caller-supplied fp32 logits */
/* Expert path (default: bf16 streams its weights below T*K = E/2 and uses
 * grouped tiles above; MXFP4 and FP8 use grouped tiles; fp32 has one path).
 * Tile height of the grouped path (default: bf16 128 rows below T*K = 96E,
 * 256 above, 160 only on request; MXFP4 64 below 56E when H and I are multiples
 * of 512, else 128 below 32E, 256 above; FP8 128 below 120E, 256 above, an
 * expert's last tile holding up to 288).  Every tile
 * height gives bit-identical outputs; the two paths agree within the layer
 * tolerance (they sum in different orders, and bf16 streaming keeps y in
 * fp32).  The flags exist for measurement and tests; at most one of the
 * BEAM_TILE_* flags, and not both path flags (else BEAM_ERR_INVALID_ARG). */
#define BEAM_PATH_STREAM (1u << 1)     /* force the weight-streaming expert path (bf16, MXFP4) */
#define BEAM_PATH_GROUPED (1u << 2)    /* force the tiled grouped-GEMM expert path */
#define BEAM_TILE_128 (1u << 3)        /* grouped path: force 128-row M tiles */
#define BEAM_TILE_256 (1u << 4)        /* grouped path: force 256-row M tiles (FP8: no 32-row
                                          extension of an expert's last tile) */
#define BEAM_TILE_160 (1u << 5)        /* bf16 grouped path: force 160-row M tiles (MXFP4 and
                                          FP8: the 256-row form) */
#define BEAM_TILE_64 (1u << 6)         /* MXFP4 grouped path: force 64-slot tiles (bf16 and
                                          FP8: the 128-row form) */

typedef struct {
  int32_t hidden;           /* H: 5120 for Beam */
  int32_t intermediate;     /* I: 2560 */
  int32_t n_experts;        /* E: 256 */
  int32_t n_groups;         /* G: 8; group g = experts [g*E/G, (g+1)*E/G) */
  int32_t topk_groups;      /* TG: 4 */
  int32_t top_k;            /* K: 8 */
  int32_t group_score_topn; /* 1 or 2 best biased scores summed per group: 2 */
  float routed_scale;       /* 2.5 */
  int32_t act_dtype;        /* dtype of x and out: BEAM_F32 or BEAM_BF16 */
  int32_t weight_dtype;     /* BEAM_F32 (needs act F32), BEAM_BF16, BEAM_FP8_E4M3, BEAM_MXFP4 */
  uint32_t flags;           /* BEAM_* flags above */
} beam_moe_desc;

/* Text for a beam_status value.  Never NULL; static storage. */
const char* beam_status_string(int status);

/* Host-only check of a descriptor and token count: makes no HIP call.
 * Supported: 1 <= E <= 1024, E % G == 0, E/G <= 64, 1 <= TG <= G,
 * 1 <= K <= min(16, TG*E/G), group_score_topn in {1,2} and <= E/G,
 * H % 128 == 0 and I % 128 == 0, routed_scale finite and > 0, T >= 0,
 * T*K*max(H, I) < 2^31 (52,428 tokens for the Beam layer), 2*I*H < 2^31
 * (one expert's gate/up matrix is addressed with 32-bit offsets).  Returns
 * BEAM_OK or the first error found. */
int beam_moe_validate(const beam_moe_desc* desc, int64_t T);

/* Bytes of workspace beam_moe_forward / beam_moe_route need for T tokens.
 * Writes 0 for T == 0.  Returns beam_moe_validate's status. */
int beam_moe_workspace_bytes(const beam_moe_desc* desc, int64_t T,
                             size_t* bytes);

/* Router only (the steps before the experts): logits x W_r^T, sigmoid
 * scores, the selection bias, group scores, the kept groups, the top K and
 * the normalised, scaled weights.  "Hugging Face releases Beam ..." (MoE
 * paragraph: 8 groups of 32 experts, best 4 groups, top 8); "Reflection
 * Releases Beam ...", section "Where Beam Saves and Where the Memory Bill
 * Comes In" (DeepSeek-V3 group-limited sigmoid router, weights normalised
 * and scaled by 2.5); "Reflection AI Introduces Beam ..." (load-balancing
 * paragraph: the bias steers selection only).
 *   x         device [T, H] act_dtype; unused with BEAM_ROUTE_LOGITS_IN
 *   w_router  device [E, H] fp32; unused with BEAM_ROUTE_LOGITS_IN
 *   bias      device [E] fp32 selection bias, or NULL for zero
 *   logits    device [T, E] fp32: written with the router logits, or read
 *             with BEAM_ROUTE_LOGITS_IN; may be NULL without that flag
 *   topk_idx  device [T, K] int32: expert ids in rank order
 *   topk_w    device [T, K] fp32: routing weights (sum to routed_scale)
 * Given identical fp32 logits the indices and weights are bitwise identical
 * to the routing specification: sigmoid rounded from a fixed binary64
 * evaluation, binary32 sums, ties broken towards the lower index. */
int beam_moe_route(const beam_moe_desc* desc, int64_t T, const void* x,
                   const float* w_router, const float* bias, float* logits,
                   int32_t* topk_idx, float* topk_w, void* workspace,
                   size_t ws_bytes, void* stream);

/* Token permutation for a given routing (the dispatch between router and
 * experts): a stable counting sort of the T*K assignments by expert.  The
 * pages route each token to 8 of 256 experts ("Hugging Face releases Beam
 * ...", MoE paragraph) and leave the dispatch to the implementation ("Beam
 * Turns Frontier-Scale Openness Into an Infrastructure Decision", section
 * "Sparse compute still requires dense planning": each token's rows have to
 * reach the experts it selected, which this grouping by expert provides).
 *   topk_idx    device [T, K] int32, each row K distinct ids in [0, E)
 *   counts      device [E] int32: assignments per expert
 *   offsets     device [E+1] int32: exclusive prefix sum of counts
 *   slot_token  device [T*K] int32: token of each slot; the slots of expert
 *               e are [offsets[e], offsets[e+1]) in increasing token order
 *   slot_of     device [T*K] int32: slot of assignment (t, k)
 * Uses the workspace (beam_moe_workspace_bytes). */
int beam_moe_permute(const beam_moe_desc* desc, int64_t T,
                     const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                     int32_t* slot_token, int32_t* slot_of, void* workspace,
                     size_t ws_bytes, void* stream);

/* Per-row, per-128-column dynamic e4m3 quantisation (the FP8 variant's
 * activation recipe): for each block, scale = amax / 448 in binary32 (1 for
 * an all-zero block), code = e4m3(v / scale) with a binary32 division,
 * round to nearest even, saturating to +-448.
 *   v       device [rows, cols] in `dtype` (BEAM_F32 or BEAM_BF16)
 *   q       device [rows, cols] uint8 codes
 *   scales  device [rows, cols/128] fp32
 * cols % 128 == 0.  No workspace. */
int beam_moe_quant_e4m3(int64_t rows, int64_t cols, int32_t dtype,
                        const void* v, uint8_t* q, float* scales, void* stream);

/* Per-row MXFP8 quantisation (the MXFP4 variant's activation recipe, OCP
 * Microscaling layout): for each block of 32 columns, x = the smallest
 * integer with amax / 2^x <= 448, clamped to [-127, 127] (-127 for an
 * all-zero block), code = e4m3(v * 2^-x) (exact scaling, round to nearest
 * even), scale byte x + 127.  (OCP's own rule, floor(log2(amax)) - 8, can
 * saturate the block maximum; this one never does.)
 *   v       device [rows, cols] in `dtype` (BEAM_F32 or BEAM_BF16)
 *   q       device [rows, cols] uint8 codes
 *   scales  device [rows, cols/32] uint8 E8M0
 * cols % 128 == 0.  No workspace. */
int beam_moe_quant_mxfp8(int64_t rows, int64_t cols, int32_t dtype,
                         const void* v, uint8_t* q, uint8_t* scales, void* stream);

/* The whole block: router, K SwiGLU experts per token and the weighted
 * combine ("Hugging Face releases Beam ...", MoE paragraph: SwiGLU
 * intermediate 2,560 on hidden 5,120; "Reflection Releases Beam ...",
 * section "Where Beam Saves and Where the Memory Bill Comes In": no shared
 * expert; "Reflection Beam", section "Where to run it", and the checkpoint
 * paragraph of "Hugging Face releases Beam ...": the FP8 and 4-bit
 * checkpoint forms).
 *   x          device [T, H] act_dtype
 *   w_router   device [E, H] fp32 (unused with BEAM_ROUTE_LOGITS_IN)
 *   bias       device [E] fp32 or NULL
 *   w_gate_up  device [E, 2I, H] weight_dtype: rows 0..I-1 gate, I..2I-1 up
 *              (MXFP4: [E, 2I, H/2] bytes)
 *   s_gate_up  device block scales, NULL for f32/bf16 weights: FP8 fp32
 *              [E, 2I/128, H/128], positive; MXFP4 E8M0 bytes [E, 2I, H/32]
 *   w_down     device [E, H, I] weight_dtype (MXFP4: [E, H, I/2] bytes)
 *   s_down     as s_gate_up: FP8 fp32 [E, H/128, I/128]; MXFP4 bytes [E, H, I/32]
 *   out        device [T, H] act_dtype
 *   topk_idx, topk_w  device [T, K] outputs of the router, or NULL
 *   logits     device [T, E] fp32: output, or input with BEAM_ROUTE_LOGITS_IN;
 *              may be NULL without that flag
 * FP8 weights also quantise x and h per token per 128 channels
 * (beam_moe_quant_e4m3's recipe) and run e4m3 matrix products with binary32
 * accumulation and block scales applied per 128-deep slice.  MXFP4 weights
 * quantise x and h to MXFP8 (beam_moe_quant_mxfp8's recipe) and run E2M1 x
 * E4M3 matrix products whose E8M0 block scales the matrix cores apply, with
 * binary32 accumulation. */
int beam_moe_forward(const beam_moe_desc* desc, int64_t T, const void* x,
                     const float* w_router, const float* bias,
                     const void* w_gate_up, const void* s_gate_up,
                     const void* w_down, const void* s_down, void* out,
                     int32_t* topk_idx, float* topk_w, float* logits,
                     void* workspace, size_t ws_bytes, void* stream);

/* beam_moe_forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace is instead a device array inside the
 * library, BEAM_NOALLOC_SCRATCH_BYTES bytes, of which every GPU the library
 * runs on holds its own copy until the process ends (looked up once per
 * device, on the first call with that device current).  The call allocates
 * nothing and makes no hipMalloc/hipFree.
 *   Arguments as beam_moe_forward without workspace and ws_bytes; `stream`
 *   must belong to the current device.
 *   BEAM_ERR_WORKSPACE when beam_moe_workspace_bytes(desc, T) exceeds
 *   BEAM_NOALLOC_SCRATCH_BYTES (64 MiB: bf16 Beam-layer batches up to about
 *   500 tokens, FP8 about 580, MXFP4 about 320); nothing is launched then.
 * All calls on one GPU share its array: calls that may overlap on one GPU
 * (on different streams, or from different host threads without ordering)
 * race and give undefined results.  Nothing in the array needs to start
 * cleared: every call writes what it reads.  Results are bitwise identical
 * to beam_moe_forward's. */
#define BEAM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int beam_moe_forward_noalloc(const beam_moe_desc* desc, int64_t T, const void* x,
                             const float* w_router, const float* bias,
                             const void* w_gate_up, const void* s_gate_up,
                             const void* w_down, const void* s_down, void* out,
                             int32_t* topk_idx, float* topk_w, float* logits,
                             void* stream);

/* beam_moe_forward followed, in the same combine kernel, by the step after
 * the block in a Beam layer stack: the post-sublayer RMSNorm of SandwichNorm
 * and the depth-scaled FP32 residual stream ("Reflection Beam", section
 * "Hybrid Attention and Unusual Residuals": at step k the stream is scaled
 * by sqrt((k-1)/k) and the sublayer output added with weight 1/sqrt(k);
 * SandwichNorm and FP32 residual accumulation from the pretraining paragraph
 * of "Reflection AI Introduces Beam ...").  Per token t, with o the fp32
 * block output before any rounding:
 *   residual[t] = sqrt((k-1)/k) * residual[t]
 *               + (1/sqrt(k)) * o / sqrt(mean(o^2) + eps) * norm_weight
 *   norm_weight  device [H] fp32 (the norm's weights; the pages give none)
 *   eps          >= 0 and finite (not on the pages; 1e-6 is usual)
 *   step         k >= 1 (k = 1 discards the incoming residual)
 *   residual     device [T, H] fp32, read and written in place
 *   out          device [T, H] act_dtype block output, or NULL to skip it
 * Other arguments as beam_moe_forward (routing outputs are not returned).
 * Requires H <= 16384 (the token's fp32 row is held in 64 KiB of LDS;
 * BEAM_ERR_UNSUPPORTED otherwise). */
int beam_moe_forward_residual(const beam_moe_desc* desc, int64_t T, const void* x,
                              const float* w_router, const float* bias,
                              const void* w_gate_up, const void* s_gate_up,
                              const void* w_down, const void* s_down,
                              const float* norm_weight, float eps, int32_t step,
                              float* residual, void* out, void* workspace,
                              size_t ws_bytes, void* stream);

/* Auxiliary-loss-free load balancing step.  The load-balancing paragraph of
 * "Reflection AI Introduces Beam ..." says Beam builds on DeepSeek-V3's
 * bias-update balancing with a cosine decay of the update speed; the rule
 * (arXiv 2412.19437 section 2.1.2) moves each expert's selection bias
 * towards balance after a batch:
 *   load_e = #{(t, k) : topk_idx[t, k] == e}
 *   bias[e] = bias[e] + gamma * sign(T*K/E - load_e)
 * with the sign decided exactly in integers (load_e*E against T*K; sign 0
 * leaves the bias unchanged) and one binary32 addition.
 *   topk_idx  device [T, K] int32 (a routing, e.g. beam_moe_route's);
 *             entries outside [0, E) are not counted
 *   bias      device [E] fp32, updated in place
 * gamma >= 0 and finite (see beam_moe_bias_gamma).  No workspace. */
int beam_moe_bias_update(const beam_moe_desc* desc, int64_t T,
                         const int32_t* topk_idx, float gamma, float* bias,
                         void* stream);

/* Update speed for step t of an n-step cosine schedule from g0 down to g1:
 * g1 + (g0 - g1) * (1 + cos(pi * t / n)) / 2, evaluated in binary64 and
 * rounded to binary32; t is clamped to [0, n].  Host only. */
float beam_moe_bias_gamma(int64_t t, int64_t n, float g0, float g1);

/* ---- measurement support ------------------------------------------------
 * A timer records a HIP event pair around every kernel a timed forward
 * launches, on the stream the kernel runs on, so tools can read per-kernel
 * durations.  It owns its events (created here, destroyed with the timer);
 * it allocates no device memory.  Not thread-safe: one timer per caller. */
typedef struct beam_moe_timer beam_moe_timer;

/* Creates a timer able to hold `capacity` kernel records.  *out is NULL on
 * error. */
int beam_moe_timer_create(int32_t capacity, beam_moe_timer** out);
void beam_moe_timer_destroy(beam_moe_timer* timer);
/* Forgets all records (keeps the events for reuse). */
void beam_moe_timer_reset(beam_moe_timer* timer);
/* Number of kernel records held. */
int32_t beam_moe_timer_count(const beam_moe_timer* timer);
/* Name and duration in milliseconds of record i; waits for its events.
 * *name points to static storage. */
int beam_moe_timer_read(beam_moe_timer* timer, int32_t i, const char** name,
                        float* ms);
/* beam_moe_forward, plus one timer record per launched kernel (records past
 * the timer's capacity are dropped).  timer may be NULL. */
int beam_moe_forward_timed(const beam_moe_desc* desc, int64_t T, const void* x,
                           const float* w_router, const float* bias,
                           const void* w_gate_up, const void* s_gate_up,
                           const void* w_down, const void* s_down, void* out,
                           int32_t* topk_idx, float* topk_w, float* logits,
                           void* workspace, size_t ws_bytes, void* stream,
                           beam_moe_timer* timer);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
