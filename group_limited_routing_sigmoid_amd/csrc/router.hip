// Router of the Beam MoE block on gfx950.
//
// The router computes sigmoid scores over the experts, adds a per-expert bias
// used only to choose experts, keeps the best groups, picks the top-K experts
// inside them and normalises their unbiased scores to sum to the routed scale
// ("Reflection Releases Beam: An Open 501B-Parameter MoE Model Under Apache
// 2.0", section "Where Beam Saves and Where the Memory Bill Comes In";
// "Hugging Face releases Beam ..." MoE paragraph; bias from the
// load-balancing paragraph of "Reflection AI Introduces Beam ...").  The
// group score is the sum of a group's best two biased scores, DeepSeek-V3's
// rule (arXiv 2412.19437, section 2.1.2), which the pages invoke.
//
// Kernels:
//   router_logits_*  logits = x W_r^T in fp32 (for many tokens the same
//                    three-term split feeds the dense tile GEMM of the
//                    grouped expert path, split over H).  With bf16 activations the
//                    fp32 router weights are split exactly into three bf16
//                    terms (hi + mid + lo), so every product is exact and the
//                    matrix cores accumulate in fp32.  The reduction over H
//                    may be split into `ks` partial sums for parallelism.
//   router_select    one wavefront per token: sums the partials in a fixed
//                    order, then routes in binary32 exactly as specified
//                    (sigmoid from a fixed binary64 evaluation, ties to the
//                    lower index), so indices and weights are bitwise
//                    reproducible from the fp32 logits.
//
// This translation unit is compiled with -ffp-contract=off.
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

// ---- logits: bf16 activations, bf16x3 split of fp32 weights, MFMA -------

__device__ __forceinline__ void split3(const float* w, bf16x8& hi, bf16x8& mid,
                                       bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = w[j];
    const bf16 h = static_cast<bf16>(v);
    const float r1 = v - static_cast<float>(h);
    const bf16 m = static_cast<bf16>(r1);
    const float r2 = r1 - static_cast<float>(m);
    hi[j] = h;
    mid[j] = m;
    lo[j] = static_cast<bf16>(r2);
  }
}

// grid (ceil(T/32), ceil(E/64), ks), four waves: 32 tokens x 64 experts (32
// in the last block when E % 64 == 32) over columns [z*kchunk, (z+1)*kchunk)
// of H.  Wave w takes the w-th quarter of those columns; the four partial
// tiles meet in LDS and are added in wave order.  With few tokens the
// kernel is bound by how much of W_r is in flight, so each wave issues the
// loads of four 16-column steps before their products.
constexpr int kLgWaves = 4;

__global__ __launch_bounds__(kLgWaves * kWave) void router_logits_mfma(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ part, int64_t T, int H, int E, int kchunk) {
  __shared__ float red[kLgWaves - 1][2][16][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int e0 = blockIdx.y * 64;
  const int z = blockIdx.z;
  const int kq = kchunk / kLgWaves;
  const int kb = z * kchunk + wave * kq + 8 * (lane / 32);
  int64_t tr = t0 + (lane % 32);
  if (tr > T - 1) tr = T - 1;
  const uint16_t* xp = x + tr * H + kb;
  // without a second 32-expert half the wave reads the first half twice and
  // stores one (keeps the loop free of branches)
  const bool has1 = e0 + 32 < E;  // wave-uniform
  const float* wp0 = wr + static_cast<int64_t>(e0 + lane % 32) * H + kb;
  const float* wp1 = wr + static_cast<int64_t>(has1 ? e0 + 32 + lane % 32 : e0 + lane % 32) * H + kb;
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll 4
  for (int k = 0; k < kq; k += 16) {
    const bf16x8 a = as_bf16x8(ld16(xp + k));
    float w0[8], w1[8];
    *reinterpret_cast<u32x4*>(w0) = ld16(wp0 + k);
    *reinterpret_cast<u32x4*>(w0 + 4) = ld16(wp0 + k + 4);
    *reinterpret_cast<u32x4*>(w1) = ld16(wp1 + k);
    *reinterpret_cast<u32x4*>(w1 + 4) = ld16(wp1 + k + 4);
    bf16x8 h0, m0, l0, h1, m1, l1;
    split3(w0, h0, m0, l0);
    split3(w1, h1, m1, l1);
    acc0 = mfma32x32x16(a, l0, acc0);
    acc1 = mfma32x32x16(a, l1, acc1);
    acc0 = mfma32x32x16(a, m0, acc0);
    acc1 = mfma32x32x16(a, m1, acc1);
    acc0 = mfma32x32x16(a, h0, acc0);
    acc1 = mfma32x32x16(a, h1, acc1);
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red[wave - 1][0][r][lane] = acc0[r];
      red[wave - 1][1][r][lane] = acc1[r];
    }
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kLgWaves - 1; ++w) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = acc0[r] + red[w][0][r][lane];
      acc1[r] = acc1[r] + red[w][1][r][lane];
    }
  }
  float* out = part + static_cast<int64_t>(z) * T * E;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t t = t0 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
    if (t < T) {
      out[t * E + e0 + lane % 32] = acc0[r];
      if (has1) out[t * E + e0 + 32 + lane % 32] = acc1[r];
    }
  }
}

// ---- exact three-term bf16 split of the fp32 router matrix ---------------
// w3 [E, 3H]: row e = [smallest term | middle term | bf16 rounding of W_r[e]];
// the three add up to W_r[e] exactly.
__global__ __launch_bounds__(256) void router_split(const float* __restrict__ wr,
                                                    uint16_t* __restrict__ w3, int E, int H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(E) * H) return;
  const int64_t e = i / H, k = i % H;
  const float v = wr[i];
  const bf16 h = static_cast<bf16>(v);
  const float r1 = v - static_cast<float>(h);
  const bf16 m = static_cast<bf16>(r1);
  const float r2 = r1 - static_cast<float>(m);
  uint16_t* row = w3 + e * 3 * H;
  row[k] = __builtin_bit_cast(uint16_t, static_cast<bf16>(r2));
  row[H + k] = __builtin_bit_cast(uint16_t, m);
  row[2 * H + k] = __builtin_bit_cast(uint16_t, h);
}

// ---- logits: generic fp32 dot products (fp32 activations, small layers) --

__global__ __launch_bounds__(256) void router_logits_valu(
    const void* __restrict__ x, int x_bf16, const float* __restrict__ wr,
    float* __restrict__ part, int64_t T, int H, int E, int kchunk) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int z = blockIdx.y;
  if (i >= T * E) return;
  const int64_t t = i / E;
  const int e = static_cast<int>(i % E);
  const int k0 = z * kchunk;
  float acc = 0.0f;
  for (int k = k0; k < k0 + kchunk; ++k) {
    const float xv = x_bf16
        ? bf16_bits_to_f32(static_cast<const uint16_t*>(x)[t * H + k])
        : static_cast<const float*>(x)[t * H + k];
    acc = __builtin_fmaf(xv, wr[static_cast<int64_t>(e) * H + k], acc);
  }
  part[static_cast<int64_t>(z) * T * E + i] = acc;
}

// ---- routing --------------------------------------------------------------

// sigmoid32(l) = 1/(1+e^-l) evaluated in binary64 and rounded once to
// binary32.  e^z: Cody & Waite reduction z = n ln2 + r (ln2 as a 32-bit head
// plus a tail), then the degree-13 Taylor polynomial of e^r in Horner form
// with fused multiply-adds; coefficients are the binary64 roundings of 1/j!.
// Every step is an IEEE-exact binary64 operation, so any conforming
// evaluation of this sequence returns the same bits.
__device__ __forceinline__ float sigmoid32(float l) {
  if (l <= -104.0f) return 0.0f;
  if (l >= 40.0f) return 1.0f;
  const double z = -static_cast<double>(l);
  const double n = __builtin_rint(z * 0x1.71547652b82fep+0);
  double r = __builtin_fma(-n, 0x1.62e42feep-1, z);
  r = __builtin_fma(-n, 0x1.a39ef35793c76p-33, r);
  double p = 0x1.6124613a86d09p-33;          // 1/13!
  p = __builtin_fma(p, r, 0x1.1eed8eff8d898p-29);  // 1/12!
  p = __builtin_fma(p, r, 0x1.ae64567f544e4p-26);  // 1/11!
  p = __builtin_fma(p, r, 0x1.27e4fb7789f5cp-22);  // 1/10!
  p = __builtin_fma(p, r, 0x1.71de3a556c734p-19);  // 1/9!
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-16);  // 1/8!
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-13);  // 1/7!
  p = __builtin_fma(p, r, 0x1.6c16c16c16c17p-10);  // 1/6!
  p = __builtin_fma(p, r, 0x1.1111111111111p-7);   // 1/5!
  p = __builtin_fma(p, r, 0x1.5555555555555p-5);   // 1/4!
  p = __builtin_fma(p, r, 0x1.5555555555555p-3);   // 1/3!
  p = __builtin_fma(p, r, 0x1.0p-1);               // 1/2!
  p = __builtin_fma(p, r, 1.0);                    // 1/1!
  p = __builtin_fma(p, r, 1.0);                    // 1/0!
  const double ez = __builtin_ldexp(p, static_cast<int>(n));
  const double q = 1.0 / (1.0 + ez);
  return static_cast<float>(q);
}

// Order-preserving map of a finite binary32 to uint32 (larger float, larger
// key); +0 and -0 map to the same key after canonicalisation.
__device__ __forceinline__ uint32_t ordered(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Rank key: larger value first, then lower expert id.  0 means "not a
// candidate" and is below every real key.
__device__ __forceinline__ uint64_t rank_key(float u, int e) {
  return (static_cast<uint64_t>(ordered(u)) << 32) |
         static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(e));
}

constexpr int kSelWaves = 4;
constexpr int kMaxE = 1024;
constexpr int kMaxKs = 16;   // the plan splits the router's reduction at most 16 ways
constexpr int kMaxG = 64;

// ---- wave-wide helpers for the selection --------------------------------

// 64-bit DPP move (both halves with the same lane pattern)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, returned uniform.  Within each row of 16 lanes:
// swap neighbours, swap pairs (quad permutations), mirror the half rows,
// mirror the row; every lane then holds its row's maximum, and the four
// rows' maxima are read out lane by lane.  Needs every lane active.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = max64(v, dpp64<0xB1>(v));   // quad_perm(1, 0, 3, 2)
  v = max64(v, dpp64<0x4E>(v));   // quad_perm(2, 3, 0, 1)
  v = max64(v, dpp64<0x141>(v));  // row_half_mirror
  v = max64(v, dpp64<0x140>(v));  // row_mirror
  return max64(max64(readlane64(v, 0), readlane64(v, 16)),
               max64(readlane64(v, 32), readlane64(v, 48)));
}

// grid ceil(T/4), block 256: wave w routes token 4*blockIdx.x + w, holding
// EPL experts per lane in registers (lane l: experts l*EPL .. l*EPL+EPL-1).
// KS is 1 (one partial per logit) or kMaxKs (ks <= kMaxKs partials).  SEG:
// a group's experts are the L = gs/EPL lanes of one aligned power-of-two
// segment, so group maxima are butterflies within the segment; otherwise
// lane g scans group g's biased scores from LDS (one pad word per 32 keeps
// the scan's lanes on distinct banks).
__device__ __forceinline__ int upad(int e) { return e + (e >> 5); }

template <int EPL, int KS, bool SEG>
__global__ __launch_bounds__(256) void router_select(
    const float* __restrict__ part, int ks, int vec4, int64_t T, int E, int G,
    int TG, int K, int topn, float scale, const float* __restrict__ bias,
    float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kSelWaves + wave;
  const bool valid = t < T;   // wave-uniform
  const int64_t tc = valid ? t : T - 1;
  const int gs = E / G;
  const float ninf = -__builtin_huge_valf();

  // 1. logits (fixed-order sum of the partials), scores, biased scores.
  // Every load is issued before the first add: indices are clamped into
  // range instead of branched on, and the clamped values are not used.
  // With vec4 (E % 4 == 0: 16-byte aligned rows) a lane's experts come four
  // to a 16-byte load.
  float pz[EPL][KS], bz[EPL], sv[EPL], u[EPL];
  if (EPL % 4 == 0 && vec4) {
#pragma unroll
    for (int j = 0; j < EPL; j += 4) {
      const int e = min(lane * EPL + j, E - 4);
#pragma unroll
      for (int z = 0; z < KS; ++z) {
        const u32x4 v = ld16(part + (static_cast<int64_t>(min(z, ks - 1)) * T + tc) * E + e);
#pragma unroll
        for (int q = 0; q < 4 && j + q < EPL; ++q) pz[j + q][z] = __uint_as_float(v[q]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = min(lane * EPL + j, E - 1);
#pragma unroll
      for (int z = 0; z < KS; ++z)
        pz[j][z] = part[(static_cast<int64_t>(min(z, ks - 1)) * T + tc) * E + e];
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) bz[j] = bias ? bias[min(lane * EPL + j, E - 1)] : 0.0f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane * EPL + j;
    float l = pz[j][0];
#pragma unroll
    for (int z = 1; z < KS; ++z)
      if (z < ks) l = l + pz[j][z];
    sv[j] = sigmoid32(l);
    u[j] = e < E ? sv[j] + bz[j] : ninf;
    if (valid && e < E && logits_out) logits_out[t * E + e] = l;
  }

  // 2. group scores: sum of the topn (1 or 2) largest biased scores (a
  // repeated value counts twice).  gsc ends in lane g for group g.
  float gsc = ninf;
  if constexpr (SEG) {
    float t1 = ninf, t2 = ninf;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if (u[j] > t1) {
        t2 = t1;
        t1 = u[j];
      } else if (u[j] > t2) {
        t2 = u[j];
      }
    }
    const int L = gs / EPL;
    for (int off = 1; off < L; off <<= 1) {
      const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
      const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
      t1 = fmaxf(t1, o1);
      t2 = n2;
    }
    const float mine = (topn == 1) ? t1 : t1 + t2;
    gsc = __shfl(mine, min(lane, G - 1) * L);
  } else {
    __shared__ float u_sh[kSelWaves][kMaxE + kMaxE / 32];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane * EPL + j;
      if (e < E) u_sh[wave][upad(e)] = u[j];
    }
    __syncthreads();
    if (lane < G) {
      float t1 = ninf, t2 = ninf;
      for (int j = 0; j < gs; ++j) {
        const float v = u_sh[wave][upad(lane * gs + j)];
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
      gsc = (topn == 1) ? t1 : t1 + t2;
    }
  }
  if (!valid) return;

  // 3. keep the TG best groups (ties: lower group id): bit g of `keep`
  int rank = 0;
  for (int g = 0; g < G; ++g) {
    const float o = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsc), g));
    rank += (o > gsc) || (o == gsc && g < lane);
  }
  const uint64_t keep = __ballot(lane < G && rank < TG);

  // 4. top-K of the eligible experts by biased score, rank order
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane * EPL + j;
    key[j] = (e < E && ((keep >> (e / gs)) & 1)) ? rank_key(u[j], e) : 0;
  }
  float D = 0.0f, my_s = 0.0f;
  int my_e = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) best = max64(best, key[j]);
    best = wave_max64(best);
    // K <= TG*E/G eligible experts always remain, so best != 0; the clamp
    // only keeps the lane index below in range.
    int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    float se = sv[0];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if (lane * EPL + j == e) key[j] = 0;
      if (j == e % EPL) se = sv[j];
    }
    const float sk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, se), e / EPL));
    D = (k == 0) ? sk : D + sk;
    if (lane == k) {
      my_e = e;
      my_s = sk;
    }
  }
  // 5. weights: (s / D) * scale, two binary32 roundings
  if (lane < K) {
    const float q = my_s / D;
    idx_out[t * K + lane] = my_e;
    w_out[t * K + lane] = q * scale;
  }
}

}  // namespace

hipError_t launch_router(const Plan& p, const void* x, const float* w_router,
                         const float* bias, float* logits_out,
                         const float* logits_in, int32_t* idx, float* w,
                         void* ws, hipStream_t s, Timer* tm) {
  const float* part = logits_in;
  int ks = 1;
  if (!logits_in) {
    ks = p.ks;
    float* buf = ws_at<float>(ws, p.off_part);
    const int kchunk = p.H / ks;
    if (p.router_gemm) {
      uint16_t* w3 = ws_at<uint16_t>(ws, p.off_w3);
      const int64_t n = static_cast<int64_t>(p.E) * p.H;
      BEAM_LAUNCH(tm, "router_split", router_split, dim3(static_cast<unsigned>(ceil_div(n, 256))),
                  dim3(256), 0, s, w_router, w3, p.E, p.H);
      const hipError_t e = launch_router_gemm(p, x, w3, buf, s, tm);
      if (e != hipSuccess) return e;
    } else if (p.act == BEAM_BF16 && p.E % 32 == 0) {
      dim3 grid(static_cast<unsigned>(ceil_div(p.T, 32)), static_cast<unsigned>(ceil_div(p.E, 64)), ks);
      BEAM_LAUNCH(tm, "router_logits_mfma", router_logits_mfma, grid, dim3(kLgWaves * kWave), 0, s,
                         static_cast<const uint16_t*>(x), w_router, buf, p.T,
                         p.H, p.E, kchunk);
    } else {
      dim3 grid(static_cast<unsigned>(ceil_div(p.T * p.E, 256)), ks);
      BEAM_LAUNCH(tm, "router_logits_valu", router_logits_valu, grid, dim3(256), 0, s, x,
                         p.act == BEAM_BF16 ? 1 : 0, w_router, buf, p.T, p.H,
                         p.E, kchunk);
    }
    part = buf;
  }
  const float* lo = logits_in ? nullptr : logits_out;
  dim3 grid(static_cast<unsigned>(ceil_div(p.T, kSelWaves)));
  const int epl = static_cast<int>(ceil_div(p.E, kWave));
  const int eplp = epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : epl <= 8 ? 8 : 16;
  const int gs = p.E / p.G, seg_l = gs / eplp;
  const bool seg = gs % eplp == 0 && (seg_l & (seg_l - 1)) == 0;
  // partials live in the workspace and given logits are 16-byte aligned
  // (checked at the boundary), so rows of E % 4 == 0 floats are too
  const int vec4 = p.E % 4 == 0;
#define BEAM_SEL3(EPL, KS, SEG)                                                \
  BEAM_LAUNCH(tm, "router_select", (router_select<EPL, KS, SEG>), grid, dim3(256), 0, s, part, \
              ks, vec4, p.T, p.E, p.G, p.TG, p.K, p.topn, p.scale, bias,      \
              const_cast<float*>(lo), idx, w)
#define BEAM_SEL(EPL)                                                          \
  do {                                                                         \
    if (ks == 1) {                                                             \
      if (seg) BEAM_SEL3(EPL, 1, true); else BEAM_SEL3(EPL, 1, false);         \
    } else {                                                                   \
      if (seg) BEAM_SEL3(EPL, kMaxKs, true); else BEAM_SEL3(EPL, kMaxKs, false); \
    }                                                                          \
  } while (0)
  if (ks > kMaxKs) return hipErrorInvalidValue;
  if (eplp == 1) BEAM_SEL(1);
  else if (eplp == 2) BEAM_SEL(2);
  else if (eplp == 4) BEAM_SEL(4);
  else if (eplp == 8) BEAM_SEL(8);
  else BEAM_SEL(16);
#undef BEAM_SEL3
#undef BEAM_SEL
  return hipGetLastError();
}

}  // namespace beam
