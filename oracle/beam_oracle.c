/*
 * CPU oracle for the Beam MoE block: a plain, slow, deliberately unoptimised
 * statement of what the block computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, includes or calls it, and it shares no source with the GPU path.
 *
 * Pages cited (titles as printed; sections in quotes):
 *   [P1] "Hugging Face releases Beam, a 501B-parameter open Mixture-of-Experts
 *        model with 1M-token context" -- paragraph on the MoE block.
 *   [P2] "Reflection Releases Beam: An Open 501B-Parameter MoE Model Under
 *        Apache 2.0" -- section "Where Beam Saves and Where the Memory Bill
 *        Comes In".
 *   [P3] "Reflection Beam" -- section "What Beam is".
 *   [P4] "Reflection AI Introduces Beam: A 501B Open-Weight MoE Model With 23B
 *        Active Parameters ..." -- paragraph on load balancing.
 *   [DSV3] DeepSeek-V3 technical report (arXiv 2412.19437), section 2.1.2,
 *        invoked because [P2] and [P3] say the router follows DeepSeek-V3's
 *        group-limited scheme.  The group-score rule below (sum of the two
 *        largest biased scores per group) comes from there; the pages do not
 *        state it.
 *
 * Routing is specified exactly in IEEE binary32 (round to nearest even, no
 * contraction): given identical fp32 logits every conforming implementation
 * returns identical expert indices and weights.  The expert MLPs and the
 * combine accumulate in binary64 and are the reference the GPU's bf16/fp8
 * results are measured against.
 *
 * Parity status: the group-score rule (top-2 sum, from [DSV3]), the FP8
 * recipe (e4m3fn, per-128 fp32 scales) and the sigmoid evaluation order are
 * readings fixed by a written specification; the pages print no routing
 * example, layer output or FP8 detail.  Which of these the tests pin against
 * independent facts is listed in the oracle's Python wrapper.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define BO_F32 0
#define BO_BF16 1
#define BO_E4M3 2
#define BO_MXFP4 3

typedef struct {
  int32_t hidden;           /* H */
  int32_t intermediate;     /* I */
  int32_t n_experts;        /* E */
  int32_t n_groups;         /* G; experts 0..E/G-1 form group 0, and so on */
  int32_t topk_groups;      /* groups kept */
  int32_t top_k;            /* experts per token */
  int32_t group_score_topn; /* how many of a group's best biased scores are summed */
  float routed_scale;       /* 2.5 */
} bo_shape;

/* ------------------------------------------------------------------------ */
/* Scalar conversions                                                        */
/* ------------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, 0x7F/0xFF are NaN, largest finite 448. */
double bo_e4m3_decode(uint8_t b) {
  int sign = b >> 7, ex = (b >> 3) & 15, man = b & 7;
  double v;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9);               /* subnormal: man/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Round a binary32 value to the nearest e4m3fn value, ties to even, and
 * saturate magnitudes above 448 to +-448 ("satfinite"). */
uint8_t bo_e4m3_encode(float f) {
  if (isnan(f)) return 0x7F;
  uint8_t sign = signbit(f) ? 0x80 : 0;
  double a = fabs((double)f);
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0.015625) {                         /* below the smallest normal 2^-6 */
    double n = nearbyint(a * 512.0);          /* multiples of 2^-9, exact scaling */
    return sign | (uint8_t)n;                 /* n == 8 is the code of 2^-6 */
  }
  int e;
  double m = frexp(a, &e);                    /* a = m * 2^e, m in [0.5,1) */
  m *= 2.0;
  e -= 1;                                     /* a = m * 2^e, m in [1,2) */
  double f8 = nearbyint((m - 1.0) * 8.0);     /* exact: m has <= 24 bits */
  int man = (int)f8;
  if (man == 8) {
    man = 0;
    e += 1;
  }
  int code = ((e + 7) << 3) | man;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

/* OCP Microscaling (MX) formats, specification v1.0: FP4 E2M1 elements (1
 * sign, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN, largest 6)
 * and E8M0 shared scales (2^(s - 127)); a block is 32 consecutive values. */
double bo_e2m1_decode(uint8_t nib) {
  int sign = (nib >> 3) & 1, ex = (nib >> 1) & 3, man = nib & 1;
  double v = (ex == 0) ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -v : v;
}

/* Nearest E2M1 value, ties to the even code, magnitudes above 6 saturate. */
uint8_t bo_e2m1_encode(double v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs(v);
  if (isnan(v)) return sign | 7;
  uint8_t best = 0;
  for (uint8_t c = 1; c < 8; ++c) {
    double d = fabs(bo_e2m1_decode(c) - a), db = fabs(bo_e2m1_decode(best) - a);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return sign | best;
}

/* Shared exponent of an MX block: floor(log2(amax)) - emax_elem (2 for
 * E2M1, 8 for E4M3), clamped to the E8M0 range [-127, 127]; -127 for an
 * all-zero block.  Returns the E8M0 code (exponent + 127). */
uint8_t bo_mx_scale(double amax, int emax_elem) {
  int x = -127;
  if (amax > 0.0) {
    int e;
    frexp(amax, &e);            /* amax = m 2^e, m in [0.5, 1): floor(log2) = e - 1 */
    x = e - 1 - emax_elem;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
  }
  return (uint8_t)(x + 127);
}

/* Shared exponent of the activation recipe of the 4-bit variant (a reading:
 * the pages give no recipe for it): the smallest power of two 2^x with
 * amax / 2^x <= 448, so the block maximum never saturates, clamped to the
 * E8M0 range; -127 for an all-zero block.  Returns the E8M0 code. */
uint8_t bo_mx8_act_scale(double amax) {
  int s = bo_mx_scale(amax, 8);                   /* floor rule: amax/2^x < 512 */
  if (amax > 0.0 && s < 254 && ldexp(amax, 127 - s) > 448.0) s += 1;
  return (uint8_t)s;
}

/* MX quantisation of n values (n a multiple of 32): fmt 4 -> E2M1 codes
 * packed two per byte (even index in the low nibble) with the OCP shared
 * exponent; fmt 8 -> E4M3 codes with the activation exponent above; one E8M0
 * scale per block; elements = encode(v / 2^x) (exact scaling). */
void bo_quant_mx(const float* v, int64_t n, int fmt, uint8_t* q, uint8_t* scales) {
  for (int64_t b0 = 0; b0 < n; b0 += 32) {
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) {
      double a = fabs((double)v[b0 + j]);
      if (a > amax) amax = a;
    }
    const uint8_t s = (fmt == 4) ? bo_mx_scale(amax, 2) : bo_mx8_act_scale(amax);
    scales[b0 / 32] = s;
    for (int j = 0; j < 32; ++j) {
      const double u = ldexp((double)v[b0 + j], 127 - (int)s);
      if (fmt == 4) {
        const uint8_t c = bo_e2m1_encode(u);
        const int64_t i = b0 + j;
        if (i % 2 == 0) q[i / 2] = c; else q[i / 2] |= (uint8_t)(c << 4);
      } else {
        q[b0 + j] = bo_e4m3_encode((float)u);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Routing specification ([P1], [P2], [P3], [P4], [DSV3])                    */
/* ------------------------------------------------------------------------ */

/* sigmoid32(l) = 1/(1+e^-l), evaluated in binary64 by a fixed sequence and
 * rounded once to binary32.  e^z uses Cody & Waite's argument reduction
 * (z = n ln2 + r with ln2 split into a 32-significant-bit head and a tail)
 * and the degree-13 Taylor polynomial of e^r in Horner form with fused
 * multiply-adds; the coefficients are the binary64 roundings of 1/j!. */
static double taylor_coef[14];

/* 1/j! for j = 0..13; j! is exact in binary64 here, so each is one rounding. */
__attribute__((constructor)) static void init_taylor_coef(void) {
  double fact = 1.0;
  for (int j = 0; j < 14; ++j) {
    if (j > 0) fact *= (double)j;
    taylor_coef[j] = 1.0 / fact;
  }
}

/* The binary64 value before the final rounding (exposed so tests can bound
 * its error directly). */
double bo_sigmoid_f64(float l) {
  const double* coef = taylor_coef;
  if (l <= -104.0f) return 0.0;
  if (l >= 40.0f) return 1.0;
  const double inv_ln2 = 0x1.71547652b82fep+0; /* binary64 rounding of 1/ln2 */
  const double ln2_hi = 0x1.62e42feep-1;       /* ln2 truncated to 32 bits */
  const double ln2_lo = 0x1.a39ef35793c76p-33; /* binary64 rounding of ln2 - ln2_hi */
  double z = -(double)l;
  double n = rint(z * inv_ln2);
  double r = fma(-n, ln2_hi, z);
  r = fma(-n, ln2_lo, r);
  double p = coef[13];
  for (int j = 12; j >= 0; --j) p = fma(p, r, coef[j]);
  double ez = ldexp(p, (int)n);
  double d = 1.0 + ez;
  return 1.0 / d;
}

float bo_sigmoid32(float l) { return (float)bo_sigmoid_f64(l); }

typedef struct {
  float key;
  int idx;
} bo_ranked;

/* Larger key first; equal keys: smaller index first. */
static int cmp_desc(const void* a, const void* b) {
  const bo_ranked* x = (const bo_ranked*)a;
  const bo_ranked* y = (const bo_ranked*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Route one token from its fp32 logits.
 *   s_e = sigmoid32(l_e)                         sigmoid scores ([P2])
 *   u_e = s_e + b_e                              bias steers selection only ([P4])
 *   G_g = sum of the topn largest u in group g,  largest first ([DSV3])
 *   keep the topk_groups best groups             ([P1], [P2], [P3])
 *   pick the top_k largest u among experts of kept groups ([P1], [P2])
 *   D   = s_{i0} + s_{i1} + ... in rank order;  w_k = (s_{ik} / D) * scale ([P2])
 * Ranks order by value, then by the lower index.  Experts outside the kept
 * groups are ineligible.  kept_out (nullable) receives the kept group ids in
 * rank order.  Returns 0, or -1 if the shape cannot supply top_k experts. */
int bo_route_token(const bo_shape* sh, const float* logits, const float* bias,
                   int32_t* idx_out, float* w_out, float* s_out,
                   int32_t* kept_out) {
  const int E = sh->n_experts, G = sh->n_groups, gs = E / G;
  const int TG = sh->topk_groups, K = sh->top_k, topn = sh->group_score_topn;
  if (E % G || TG > G || K > TG * gs || topn < 1 || topn > gs) return -1;
  float* s = (float*)malloc(sizeof(float) * E);
  float* u = (float*)malloc(sizeof(float) * E);
  bo_ranked* r = (bo_ranked*)malloc(sizeof(bo_ranked) * (E > G ? E : G));
  for (int e = 0; e < E; ++e) {
    s[e] = bo_sigmoid32(logits[e]);
    u[e] = s[e] + (bias ? bias[e] : 0.0f);
  }
  /* group scores */
  bo_ranked* gr = (bo_ranked*)malloc(sizeof(bo_ranked) * G);
  for (int g = 0; g < G; ++g) {
    for (int j = 0; j < gs; ++j) {
      r[j].key = u[g * gs + j];
      r[j].idx = g * gs + j;
    }
    qsort(r, gs, sizeof(bo_ranked), cmp_desc);
    float acc = r[0].key;
    for (int j = 1; j < topn; ++j) acc = acc + r[j].key;
    gr[g].key = acc;
    gr[g].idx = g;
  }
  qsort(gr, G, sizeof(bo_ranked), cmp_desc);
  /* eligible experts of the kept groups */
  int n = 0;
  for (int k = 0; k < TG; ++k) {
    int g = gr[k].idx;
    if (kept_out) kept_out[k] = g;
    for (int j = 0; j < gs; ++j) {
      r[n].key = u[g * gs + j];
      r[n].idx = g * gs + j;
      ++n;
    }
  }
  qsort(r, n, sizeof(bo_ranked), cmp_desc);
  float D = 0.0f;
  for (int k = 0; k < K; ++k) {
    idx_out[k] = r[k].idx;
    D = (k == 0) ? s[r[k].idx] : D + s[r[k].idx];
  }
  for (int k = 0; k < K; ++k) {
    float sk = s[r[k].idx];
    float q = sk / D;
    w_out[k] = q * sh->routed_scale;
    if (s_out) s_out[k] = sk;
  }
  free(gr);
  free(r);
  free(u);
  free(s);
  return 0;
}

int bo_route(const bo_shape* sh, int64_t T, const float* logits,
             const float* bias, int32_t* idx, float* w, int32_t* kept) {
  for (int64_t t = 0; t < T; ++t) {
    int rc = bo_route_token(sh, logits + t * sh->n_experts, bias,
                            idx + t * sh->top_k, w + t * sh->top_k, NULL,
                            kept ? kept + t * sh->topk_groups : NULL);
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Activations and weights as exact binary64 values                          */
/* ------------------------------------------------------------------------ */

static double load_val(const void* base, int dtype, int64_t i) {
  if (dtype == BO_F32) return (double)((const float*)base)[i];
  if (dtype == BO_BF16) return (double)bf16_to_f32(((const uint16_t*)base)[i]);
  return bo_e4m3_decode(((const uint8_t*)base)[i]);
}

/* Per-token, per-block dynamic quantisation to e4m3 (the FP8 variant's
 * activation recipe): scale = amax / 448 in binary32, or 1 where that is
 * zero (an all-zero block, or a subnormal amax whose quotient underflows),
 * code = e4m3(v / scale) with a binary32 division, saturating (a subnormal
 * scale is coarse, so v / scale may pass 448).  Writes the codes and one
 * scale per block.  n must be a multiple of block. */
void bo_quant_e4m3(const float* v, int64_t n, int block, uint8_t* q,
                   float* scales) {
  for (int64_t b0 = 0; b0 < n; b0 += block) {
    float amax = 0.0f;
    for (int j = 0; j < block; ++j) {
      float a = fabsf(v[b0 + j]);
      if (a > amax) amax = a;
    }
    float sc = amax / 448.0f;
    if (!(sc > 0.0f)) sc = 1.0f;
    scales[b0 / block] = sc;
    for (int j = 0; j < block; ++j) q[b0 + j] = bo_e4m3_encode(v[b0 + j] / sc);
  }
}

/* Round-trip a row through MXFP8 (E4M3 elements, E8M0 per 32 values). */
static void fake_quant_row_mx(const double* in, int64_t n, double* out, float* tmpf,
                              uint8_t* tmpq, uint8_t* tmps) {
  for (int64_t i = 0; i < n; ++i) tmpf[i] = (float)in[i];
  bo_quant_mx(tmpf, n, 8, tmpq, tmps);
  for (int64_t i = 0; i < n; ++i)
    out[i] = ldexp(bo_e4m3_decode(tmpq[i]), (int)tmps[i / 32] - 127);
}

/* Binary32 -> bfloat16 (round to nearest, ties to even) -> binary32. */
static float round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) != 0x7F800000u) {       /* finite: add half an ulp, tie to even */
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
  }
  memcpy(&f, &u, 4);
  return f;
}

/* Round-trip a row through bo_quant_e4m3 and return the dequantised values.
 * bf16_first: the row is taken as binary32 values rounded to bfloat16 (the
 * precision intermediate activations are stored in) before quantising. */
static void fake_quant_row(const double* in, int64_t n, int block, double* out,
                           float* tmpf, uint8_t* tmpq, float* tmps, int bf16_first) {
  for (int64_t i = 0; i < n; ++i) tmpf[i] = bf16_first ? round_bf16((float)in[i]) : (float)in[i];
  bo_quant_e4m3(tmpf, n, block, tmpq, tmps);
  for (int64_t i = 0; i < n; ++i)
    out[i] = bo_e4m3_decode(tmpq[i]) * (double)tmps[i / block];
}

/* Router logits in binary64: logits[t,e] = sum_h x[t,h] * W_r[e,h]. */
void bo_logits(const bo_shape* sh, int64_t T, const void* x, int x_dtype,
               const float* w_router, double* out, int nthreads) {
  const int H = sh->hidden, E = sh->n_experts;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += load_val(x, x_dtype, t * H + h) * (double)w_router[(int64_t)e * H + h];
      out[t * E + e] = acc;
    }
  }
}

/* Weight element with its block scale applied.  FP8: fp32 scale arrays
 * [rows/128, cols/128] per expert.  MXFP4: codes [rows, cols/2] (even column
 * in the low nibble) and E8M0 scales [rows, cols/32] per expert. */
static double weight(const void* w, int dtype, const void* sc, int64_t e,
                     int64_t rows, int64_t cols, int64_t r, int64_t c) {
  if (dtype == BO_MXFP4) {
    const int64_t row = e * rows + r;
    const uint8_t b = ((const uint8_t*)w)[row * (cols / 2) + c / 2];
    const uint8_t s = ((const uint8_t*)sc)[row * (cols / 32) + c / 32];
    return ldexp(bo_e2m1_decode((c % 2) ? (b >> 4) : (b & 15)), (int)s - 127);
  }
  double v = load_val(w, dtype, (e * rows + r) * cols + c);
  if (dtype == BO_E4M3) {
    int64_t nb_c = cols / 128;
    v *= (double)((const float*)sc)[(e * (rows / 128) + r / 128) * nb_c + c / 128];
  }
  return v;
}

/* The block's output for a list of tokens, given their routing.
 *   For each of the token's top_k experts e ([P1], [P2]):
 *     g = x W_g[e]^T,  v = x W_u[e]^T      W_gu[e] rows 0..I-1 gate, I..2I-1 up
 *     h = silu(g) * v, silu(g) = g / (1 + e^-g)      (SwiGLU MLP)
 *     y_e = h W_d[e]^T
 *   out[t] = sum_k w_k y_{e_k}, in rank order; no shared expert ([P2]).
 * Everything in binary64.  act_quant = 1 first round-trips x (per token) and
 * h (per assignment) through the variant's activation recipe: bo_quant_e4m3
 * per 128 channels for FP8 weights, h first rounded to binary32 and then to
 * bfloat16 (the precision the bf16 path stores h in); MXFP8 (bo_quant_mx, 32
 * channels, h rounded to binary32) for MXFP4 weights.
 * tokens[n] lists which rows of x to evaluate; out is [n, H]. */
int bo_forward_tokens(const bo_shape* sh, int64_t n, const int64_t* tokens,
                      const void* x, int x_dtype, const int32_t* idx,
                      const float* w, const void* w_gate_up,
                      const void* s_gate_up, const void* w_down,
                      const void* s_down, int w_dtype, int act_quant,
                      double* out, int nthreads) {
  const int64_t H = sh->hidden, I = sh->intermediate;
  const int K = sh->top_k;
  const int64_t qb = (w_dtype == BO_MXFP4) ? 32 : 128;  /* activation block */
  if (act_quant && (H % qb || I % qb)) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = tokens[i];
    double* xr = (double*)malloc(sizeof(double) * H);
    double* hv = (double*)malloc(sizeof(double) * I);
    double* acc = (double*)calloc(H, sizeof(double));
    int64_t m = H > I ? H : I;
    float* tf = (float*)malloc(sizeof(float) * m);
    uint8_t* tq = (uint8_t*)malloc(m);
    float* ts = (float*)malloc(sizeof(float) * (m / 128 + 1));
    uint8_t* tm = (uint8_t*)malloc(m / 32 + 1);
    const int mx = w_dtype == BO_MXFP4;
    for (int64_t h = 0; h < H; ++h) xr[h] = load_val(x, x_dtype, t * H + h);
    if (act_quant && mx) fake_quant_row_mx(xr, H, xr, tf, tq, tm);
    else if (act_quant) fake_quant_row(xr, H, 128, xr, tf, tq, ts, 0);
    for (int k = 0; k < K; ++k) {
      const int64_t e = idx[t * K + k];
      for (int64_t j = 0; j < I; ++j) {
        double g = 0.0, v = 0.0;
        for (int64_t h = 0; h < H; ++h) {
          g += xr[h] * weight(w_gate_up, w_dtype, s_gate_up, e, 2 * I, H, j, h);
          v += xr[h] * weight(w_gate_up, w_dtype, s_gate_up, e, 2 * I, H, I + j, h);
        }
        hv[j] = g / (1.0 + exp(-g)) * v;
      }
      if (act_quant && mx) fake_quant_row_mx(hv, I, hv, tf, tq, tm);
      else if (act_quant) fake_quant_row(hv, I, 128, hv, tf, tq, ts, 1);
      const double wk = (double)w[t * K + k];
      for (int64_t o = 0; o < H; ++o) {
        double y = 0.0;
        for (int64_t j = 0; j < I; ++j)
          y += hv[j] * weight(w_down, w_dtype, s_down, e, H, I, o, j);
        acc[o] += wk * y;
      }
    }
    memcpy(out + i * H, acc, sizeof(double) * H);
    free(tm);
    free(ts);
    free(tq);
    free(tf);
    free(acc);
    free(hv);
    free(xr);
  }
  return 0;
}

/* Auxiliary-loss-free load balancing ([P4]: DeepSeek-V3's bias-update
 * balancing with a cosine-decayed update speed; rule from [DSV3] section
 * 2.1.2): after a batch, every expert's bias moves by gamma towards balance,
 *   b_e = b_e + gamma * sign(mean_load - load_e),  mean_load = T*K/E,
 * with sign(0) = 0 and one binary32 addition.  load_e counts the (token,
 * expert) assignments of the batch; the sign is decided exactly in integers
 * (load_e * E against T * K). */
void bo_bias_update(int E, int64_t T, int K, const int32_t* idx, float gamma,
                    float* bias) {
  int64_t* load = (int64_t*)calloc(E, sizeof(int64_t));
  for (int64_t i = 0; i < T * K; ++i) load[idx[i]] += 1;
  for (int e = 0; e < E; ++e) {
    const int64_t lhs = load[e] * E, rhs = T * K;
    const float step = (lhs < rhs) ? gamma : ((lhs > rhs) ? -gamma : 0.0f);
    bias[e] = bias[e] + step;
  }
  free(load);
}

/* Cosine decay of the update speed over a schedule of n steps ([P4] names a
 * cosine decay; the endpoints are inputs): gamma_t = g1 + (g0 - g1) * (1 +
 * cos(pi * t / n)) / 2, in binary64, rounded to binary32. */
float bo_bias_gamma(int64_t t, int64_t n, float g0, float g1) {
  const double pi = 3.14159265358979323846;
  const double c = 0.5 * (1.0 + cos(pi * (double)t / (double)n));
  return (float)((double)g1 + ((double)g0 - (double)g1) * c);
}

/* Post-block epilogue of the depth-scaled residual stream ("Reflection Beam",
 * section "Hybrid Attention and Unusual Residuals"; SandwichNorm and FP32
 * residual accumulation from the pretraining paragraph of "Reflection AI
 * Introduces Beam ..."), in binary64 for each of the T rows:
 *   n = o / sqrt(mean(o^2) + eps) * gamma      (post-sublayer RMSNorm)
 *   r = sqrt((k - 1) / k) * r + n / sqrt(k)    (step k >= 1 of the stream)
 * o [T, H] and r [T, H] binary64, gamma [H] binary32; r is updated in place. */
void bo_residual_epilogue(int64_t T, int H, const double* o, const float* gamma,
                          double eps, int k, double* r) {
  const double a = sqrt((double)(k - 1) / (double)k);
  const double b = 1.0 / sqrt((double)k);
  for (int64_t t = 0; t < T; ++t) {
    const double* ot = o + t * (int64_t)H;
    double* rt = r + t * (int64_t)H;
    double ss = 0.0;
    for (int j = 0; j < H; ++j) ss += ot[j] * ot[j];
    const double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int j = 0; j < H; ++j) rt[j] = a * rt[j] + b * (ot[j] * inv * (double)gamma[j]);
  }
}

int bo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
