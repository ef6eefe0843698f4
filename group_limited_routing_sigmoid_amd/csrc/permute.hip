// Token permutation between the router and the experts: every token goes to
// K of the E experts ("Beam Turns Frontier-Scale Openness Into an
// Infrastructure Decision", section "Sparse compute still requires dense
// planning"), so the T*K (token, expert) assignments are grouped by expert
// before the expert matrix products.  Integer work only; the result is a
// stable counting sort (slots of one expert in increasing token order), so it
// is identical on every run.
//
//   perm_rank     per block of 256 tokens: a [E x 256] bit matrix in LDS
//                 (bit t of row e set when token t chose e); per-block expert
//                 histogram = row popcounts; rank of (t, e) inside the block
//                 = popcount of row e below bit t.
//   perm_scan     one block: per-expert prefix over blocks, counts, offsets,
//                 grouped-GEMM M-tile list (with each expert's first tile)
//                 and the list of active experts.
//   perm_scatter  slot = offsets[e] + block base + rank.
//   perm_small    T <= 256 (one block of tokens): the three steps above in
//                 one workgroup, the bit matrix kept in LDS throughout (the
//                 same slots; two launches fewer for decode batches).
//   bias_update   the expert-bias balancing step on the same histogram idea
//                 ("Reflection AI Introduces Beam ...", load-balancing
//                 paragraph; DeepSeek-V3's bias-update rule).
#include "common.h"
#include "internal.h"

namespace beam {
namespace {

constexpr int kMaxE = 1024;
constexpr int kWords = kPermBlock / 32;

__global__ __launch_bounds__(kPermBlock) void perm_rank(
    const int32_t* __restrict__ idx, int64_t T, int K, int E,
    int32_t* __restrict__ hist, int32_t* __restrict__ rank) {
  __shared__ uint32_t bits[kMaxE * kWords];
  const int lt = threadIdx.x;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + lt;
  for (int i = lt; i < E * kWords; i += kPermBlock) bits[i] = 0;
  __syncthreads();
  if (t < T)
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      atomicOr(&bits[e * kWords + lt / 32], 1u << (lt % 32));
    }
  __syncthreads();
  for (int e = lt; e < E; e += kPermBlock) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popc(bits[e * kWords + w]);
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
  if (t < T)
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      int r = __popc(bits[e * kWords + lt / 32] & ((1u << (lt % 32)) - 1u));
      for (int w = 0; w < lt / 32; ++w) r += __popc(bits[e * kWords + w]);
      rank[t * K + k] = r;
    }
}

// Inclusive scans of four values at once over the 1024 threads of the
// block: within each wave by shifts of 1, 2, .., 32 lanes, then each wave
// adds the totals of the waves before it (read from LDS).  Integer sums, so
// any order gives the same result.
__device__ void block_scan4_incl(int (&v)[4]) {
  __shared__ int tot[4][kMaxE / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = __shfl_up(v[q], off);
    if (lane >= off)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += u[q];
  }
  if (lane == kWave - 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[q][wave] = v[q];
  __syncthreads();
  for (int w = 0; w < wave; ++w)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += tot[q][w];
  __syncthreads();
}

// Per expert (thread e of a 1024-thread block; experts past E count 0):
// slots, offsets, the active list, the M tiles (of bm rows, the last holding
// up to bm + xt) and the tile table, hot experts' tiles first.  Returns the
// expert's exclusive slot offset.
__device__ int expert_tables(int e, int c, int E, int bm, int xt, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ meta,
                             int32_t* __restrict__ active, int32_t* __restrict__ tt) {
  __shared__ int n_hot;
  const int nt = (c <= 0) ? 0 : max(1, (c - xt + bm - 1) / bm);
  const int hot = nt >= kHotTiles;
  int v[4] = {c, nt, c > 0, hot ? nt : 0};
  block_scan4_incl(v);
  if (threadIdx.x == kMaxE - 1) n_hot = v[3];
  __syncthreads();
  const int off = v[0] - c;
  const int t_before = v[1] - nt, hot_before = v[3] - (hot ? nt : 0);
  const int pos = hot ? hot_before : n_hot + (t_before - hot_before);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    if (c > 0) active[v[2] - 1] = e;
    tt[e] = pos;
    tt[tt_count(E) + e] = nt;
    for (int t = 0; t < nt; ++t) tt[tt_expert(E) + pos + t] = e;
  }
  if (e == E - 1) {
    offsets[E] = v[0];
    tt[E] = v[1];
    meta[kMetaTiles] = v[1];
    meta[kMetaActive] = v[2];
    meta[kMetaHot] = n_hot;
  }
  return off;
}

// one block of 1024 threads; thread e handles expert e
__global__ __launch_bounds__(kMaxE) void perm_scan(
    const int32_t* __restrict__ hist, int64_t nb, int E, int bm, int xt,
    int32_t* __restrict__ base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ meta,
    int32_t* __restrict__ active, int32_t* __restrict__ tile_off) {
  const int e = threadIdx.x;
  int c = 0;
  if (e < E) {
    // eight blocks' counts loaded before they are added
    int64_t b = 0;
    for (; b + 8 <= nb; b += 8) {
      int hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) hv[j] = hist[(b + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        base[(b + j) * E + e] = c;
        c += hv[j];
      }
    }
    for (; b < nb; ++b) {
      base[b * E + e] = c;
      c += hist[b * E + e];
    }
  }
  expert_tables(e, c, E, bm, xt, counts, offsets, meta, active, tile_off);
}

__global__ __launch_bounds__(kPermBlock) void perm_scatter(
    const int32_t* __restrict__ idx, int64_t T, int K, int E,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token,
    int32_t* __restrict__ slot_of) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + threadIdx.x;
  if (t >= T) return;
  for (int k = 0; k < K; ++k) {
    const int e = idx[t * K + k];
    const int slot = offsets[e] + base[static_cast<int64_t>(blockIdx.x) * E + e] +
                     rank[t * K + k];
    slot_token[slot] = static_cast<int32_t>(t);
    slot_of[t * K + k] = slot;
  }
}

// one block of 1024 threads: thread t < T marks and places token t, thread
// e < E counts and scans expert e
__global__ __launch_bounds__(kMaxE) void perm_small(
    const int32_t* __restrict__ idx, int T, int K, int E, int bm, int xt,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ meta, int32_t* __restrict__ active,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ slot_token,
    int32_t* __restrict__ slot_of) {
  __shared__ uint32_t bits[kMaxE * kWords];
  __shared__ int off_sh[kMaxE];
  const int i = threadIdx.x;
  for (int j = i; j < E * kWords; j += kMaxE) bits[j] = 0;
  __syncthreads();
  if (i < T)
    for (int k = 0; k < K; ++k) {
      const int e = idx[i * K + k];
      atomicOr(&bits[e * kWords + i / 32], 1u << (i % 32));
    }
  __syncthreads();
  int c = 0;
  if (i < E)
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popc(bits[i * kWords + w]);
  const int off = expert_tables(i, c, E, bm, xt, counts, offsets, meta, active, tile_off);
  if (i < E) off_sh[i] = off;
  __syncthreads();
  if (i < T)
    for (int k = 0; k < K; ++k) {
      const int e = idx[i * K + k];
      int r = __popc(bits[e * kWords + i / 32] & ((1u << (i % 32)) - 1u));
      for (int w = 0; w < i / 32; ++w) r += __popc(bits[e * kWords + w]);
      const int slot = off_sh[e] + r;
      slot_token[slot] = i;
      slot_of[i * K + k] = slot;
    }
}

// Expert-bias balancing step: one workgroup; integer histogram in LDS, then
// bias[e] += gamma * sign(T*K - load_e*E) with the sign taken in integers.
__global__ __launch_bounds__(kMaxE) void bias_update(
    const int32_t* __restrict__ idx, int64_t TK, int E, float gamma,
    float* __restrict__ bias) {
  __shared__ int load[kMaxE];
  for (int e = threadIdx.x; e < E; e += kMaxE) load[e] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < TK; i += kMaxE) {
    const uint32_t e = static_cast<uint32_t>(idx[i]);
    if (e < static_cast<uint32_t>(E)) atomicAdd(&load[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMaxE) {
    const int64_t lhs = static_cast<int64_t>(load[e]) * E;
    const float step = (lhs < TK) ? gamma : ((lhs > TK) ? -gamma : 0.0f);
    bias[e] = bias[e] + step;
  }
}

}  // namespace

hipError_t launch_bias_update(const Plan& p, const int32_t* idx, float gamma,
                              float* bias, hipStream_t s, Timer* tm) {
  BEAM_LAUNCH(tm, "bias_update", bias_update, dim3(1), dim3(kMaxE), 0, s, idx,
              p.S, p.E, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_permute(const Plan& p, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* slot_token,
                          int32_t* slot_of, void* ws, hipStream_t s, Timer* tm) {
  int32_t* hist = ws_at<int32_t>(ws, p.off_hist);
  int32_t* base = ws_at<int32_t>(ws, p.off_base);
  int32_t* rank = ws_at<int32_t>(ws, p.off_rank);
  const unsigned nb = static_cast<unsigned>(p.nb);
  if (p.T <= kPermBlock) {
    BEAM_LAUNCH(tm, "perm_small", perm_small, dim3(1), dim3(kMaxE), 0, s, idx,
                static_cast<int>(p.T), p.K, p.E, p.bm, p.xt, counts, offsets,
                ws_at<int32_t>(ws, p.off_meta), ws_at<int32_t>(ws, p.off_active),
                ws_at<int32_t>(ws, p.off_tile_off), slot_token, slot_of);
    return hipGetLastError();
  }
  BEAM_LAUNCH(tm, "perm_rank", perm_rank, dim3(nb), dim3(kPermBlock), 0, s, idx, p.T,
                     p.K, p.E, hist, rank);
  BEAM_LAUNCH(tm, "perm_scan", perm_scan, dim3(1), dim3(kMaxE), 0, s, hist, p.nb, p.E,
                     p.bm, p.xt, base, counts, offsets,
                     ws_at<int32_t>(ws, p.off_meta),
                     ws_at<int32_t>(ws, p.off_active),
                     ws_at<int32_t>(ws, p.off_tile_off));
  BEAM_LAUNCH(tm, "perm_scatter", perm_scatter, dim3(nb), dim3(kPermBlock), 0, s, idx, p.T,
                     p.K, p.E, base, rank, offsets, slot_token, slot_of);
  return hipGetLastError();
}

}  // namespace beam
