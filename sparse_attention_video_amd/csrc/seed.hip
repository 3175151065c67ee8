// k-means++ cold seeding: svgear_kmeanspp.
//
// SVG2 summary, "Efficient System-Algorithm Co-Design": a cold start takes
// k-means++ initial centroids (later denoising steps reuse the cache).  The
// seeds are D^2 samples: the first is uniform, each later one is drawn with
// probability proportional to the squared distance to the nearest seed so far.
//
// The caller supplies the randomness as one uniform 64-bit word per seed, and
// every decision is made exactly, so any implementation that follows the same
// rules picks the same tokens:
//   * D^2 of a token is summed over the coordinates in index order in fp64,
//     one rounding per product and per sum (no fused multiply-add);
//   * weights are the integers floor(D^2 * 2^k), k the largest exponent with
//     N * max D^2 * 2^k < 2^62 for the distances to the first seed (later
//     distances only shrink), so every prefix sum is exact in uint64;
//   * seed c is the first token whose inclusive prefix exceeds
//     floor(word_c * total / 2^64); seed 0 (and any draw with total 0) is
//     token floor(word * N / 2^64).
//
// One round per seed: the distance kernel updates every token's nearest-seed
// distance against the newest seed and writes per-tile weight sums; the select
// kernel scans the tile sums, finds the tile and then the token, and copies
// the token's row into the centroid table.
#include <float.h>

#include "common.h"
#include "host.h"

namespace svg {

constexpr int PP_TILE = 256;  // tokens per distance workgroup (one per thread)

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, SV_WAVE);
  return v;
}

// exclusive scan of one uint64 per thread over a 256-thread block
__device__ __forceinline__ uint64_t block_exscan_u64(uint64_t v, uint64_t* s_w /* >= 4 */, uint64_t* total) {
  const int lane = lane_id(), w = wave_id();
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < SV_WAVE; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, SV_WAVE);
    if (lane >= o) x += y;
  }
  if (lane == SV_WAVE - 1) s_w[w] = x;
  __syncthreads();
  uint64_t base = 0;
  for (int i = 0; i < w; ++i) base += s_w[i];
  *total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  __syncthreads();
  return base + x - v;
}

// D^2 in the fixed order (coordinates ascending, separate product and sum
// roundings) of one row held in LDS
template <typename T, int D>
__device__ __forceinline__ double d2_in_order(const char* row, const double* __restrict__ c) {
#pragma clang fp contract(off)
  double acc = 0.0;
  constexpr int PER = 16 / sizeof(T);
#pragma unroll 4
  for (int d0 = 0; d0 < D; d0 += PER) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(row + d0 * sizeof(T));
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const double diff = (double)to_f32(v[e]) - c[d0 + e];
      const double sq = diff * diff;
      acc = acc + sq;
    }
  }
  return acc;
}

// LDS row stride of a staged tile: the row plus 16 bytes, so the 16-byte reads
// of 16 consecutive rows at one column fall on 16 different 4-bank groups
template <typename T, int D>
constexpr int pp_stride() { return D * (int)sizeof(T) + 16; }

__device__ __forceinline__ uint64_t pp_weight(double d2, int k) {
  return (uint64_t)floor(ldexp(d2, k));
}

// seed 0: token floor(word_0 * N / 2^64) of every (batch, head)
template <typename T, int D>
__global__ void __launch_bounds__(64) pp_first_kernel(const T* __restrict__ x, int N, int C,
                                                      const uint64_t* __restrict__ words, float* __restrict__ cent,
                                                      int32_t* __restrict__ chosen) {
  const int bh = blockIdx.x;
  const int t = (int)__umul64hi(words[(size_t)bh * C], (uint64_t)N);
  const T* row = x + ((size_t)bh * N + t) * D;
  for (int d = threadIdx.x; d < D; d += 64) cent[(size_t)bh * C * D + d] = to_f32(row[d]);
  if (threadIdx.x == 0 && chosen) chosen[(size_t)bh * C] = t;
}

// FIRST: mind = D^2 to seed 0 and the per-tile maximum.  Otherwise: mind =
// min(mind, D^2 to seed c - 1) and the per-tile sum of the weights.
// The tile's rows are contiguous in x: they are staged through LDS with
// coalesced 16-byte loads, then each thread sums its own row.
template <typename T, int D, bool FIRST>
__global__ void __launch_bounds__(PP_TILE) pp_dist_kernel(const T* __restrict__ x, int N, int C, int c,
                                                          const float* __restrict__ cent, double* __restrict__ mind,
                                                          const int* __restrict__ kexp, double* __restrict__ tmax,
                                                          uint64_t* __restrict__ tsum, int ntiles) {
  constexpr int RB = D * (int)sizeof(T), ST = pp_stride<T, D>(), CPR = RB / 16;
  __shared__ __attribute__((aligned(16))) char s_x[PP_TILE * ST];
  __shared__ double s_c[D];
  __shared__ double s_m[4];
  __shared__ uint64_t s_s[4];
  const int bh = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const float* cr = cent + ((size_t)bh * C + (FIRST ? 0 : c - 1)) * D;
  for (int d = tid; d < D; d += PP_TILE) s_c[d] = (double)cr[d];
  const int t0 = tile * PP_TILE;
  const int rows = min(PP_TILE, N - t0);
  const char* src = reinterpret_cast<const char*>(x + ((size_t)bh * N + t0) * D);
  // all of a thread's 16-byte loads of a batch are issued before any is stored
  constexpr int PER = PP_TILE * CPR / PP_TILE;  // chunks per thread (CPR)
  constexpr int BATCH = PER < 16 ? PER : 16;
#pragma unroll
  for (int b0 = 0; b0 < PER; b0 += BATCH) {
    u32x4 v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int u = tid + (b0 + i) * PP_TILE;
      v[i] = u < rows * CPR ? *reinterpret_cast<const u32x4*>(src + (size_t)u * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int u = tid + (b0 + i) * PP_TILE;
      if (u < rows * CPR) {
        const int r = u / CPR, cc = u - r * CPR;
        *reinterpret_cast<u32x4*>(s_x + r * ST + cc * 16) = v[i];
      }
    }
  }
  __syncthreads();
  const int t = t0 + tid;
  double d2 = 0.0;
  if (t < N) {
    d2 = d2_in_order<T, D>(s_x + tid * ST, s_c);
    double* m = mind + (size_t)bh * N + t;
    if (!FIRST) d2 = fmin(*m, d2);
    *m = d2;
  }
  if constexpr (FIRST) {
    double v = d2;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmax(v, shfl_xor_d(v, o));
    if (lane_id() == 0) s_m[wave_id()] = v;
    __syncthreads();
    if (tid == 0) tmax[(size_t)bh * ntiles + tile] = fmax(fmax(s_m[0], s_m[1]), fmax(s_m[2], s_m[3]));
  } else {
    const uint64_t w = t < N ? pp_weight(d2, kexp[bh]) : 0;
    const uint64_t s = wave_sum_u64(w);
    if (lane_id() == 0) s_s[wave_id()] = s;
    __syncthreads();
    if (tid == 0) tsum[(size_t)bh * ntiles + tile] = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
  }
}

// k from the distances to seed 0: the largest k with N * max D^2 * 2^k < 2^62
__global__ void __launch_bounds__(256) pp_scale_kernel(const double* __restrict__ tmax, int ntiles, int N,
                                                       int* __restrict__ kexp) {
  __shared__ double s_m[4];
  const int bh = blockIdx.x;
  double v = 0.0;
  for (int i = threadIdx.x; i < ntiles; i += 256) v = fmax(v, tmax[(size_t)bh * ntiles + i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, shfl_xor_d(v, o));
  if (lane_id() == 0) s_m[wave_id()] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double m = fmax(fmax(s_m[0], s_m[1]), fmax(s_m[2], s_m[3]));
    int e = 0;
    if (m > 0.0) frexp((double)N * m, &e);
    kexp[bh] = m > 0.0 ? 62 - e : 0;
  }
}

// per-tile weight sums from the stored distances (the round after FIRST)
__global__ void __launch_bounds__(PP_TILE) pp_weights_kernel(const double* __restrict__ mind, int N,
                                                             const int* __restrict__ kexp,
                                                             uint64_t* __restrict__ tsum, int ntiles) {
  __shared__ uint64_t s_s[4];
  const int bh = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const int t = tile * PP_TILE + tid;
  const uint64_t w = t < N ? pp_weight(mind[(size_t)bh * N + t], kexp[bh]) : 0;
  const uint64_t s = wave_sum_u64(w);
  if (lane_id() == 0) s_s[wave_id()] = s;
  __syncthreads();
  if (tid == 0) tsum[(size_t)bh * ntiles + tile] = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
}

// seed c of every (batch, head): the tile, then the token, whose prefix range
// holds the target; the row is copied into the centroid table
template <typename T, int D>
__global__ void __launch_bounds__(PP_TILE) pp_select_kernel(const T* __restrict__ x, int N, int C, int c,
                                                            const uint64_t* __restrict__ words,
                                                            const double* __restrict__ mind,
                                                            const int* __restrict__ kexp,
                                                            const uint64_t* __restrict__ tsum, int ntiles,
                                                            float* __restrict__ cent, int32_t* __restrict__ chosen) {
  __shared__ uint64_t s_w[4];
  __shared__ int s_tile;
  __shared__ uint64_t s_base;
  __shared__ int s_tok;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const uint64_t word = words[(size_t)bh * C + c];
  const uint64_t* ts = tsum + (size_t)bh * ntiles;
  // each thread owns a contiguous run of tiles
  const int per = (ntiles + PP_TILE - 1) / PP_TILE;
  const int j0 = min(ntiles, tid * per), j1 = min(ntiles, j0 + per);
  uint64_t mine = 0;
  for (int j = j0; j < j1; ++j) mine += ts[j];
  uint64_t total;
  uint64_t run = block_exscan_u64(mine, s_w, &total);
  if (tid == 0) { s_tile = -1; s_tok = -1; }
  __syncthreads();
  int tok;
  if (total == 0) {
    tok = (int)__umul64hi(word, (uint64_t)N);
  } else {
    const uint64_t target = __umul64hi(word, total);
    for (int j = j0; j < j1; ++j) {
      const uint64_t sj = ts[j];
      if (run <= target && target - run < sj) { s_tile = j; s_base = run; }
      run += sj;
    }
    __syncthreads();
    // the tile sums add up to total > target, so exactly one tile holds it;
    // the guards only keep a corrupted workspace from reading out of range
    const int j = max(s_tile, 0);
    const uint64_t local = target - s_base;
    const int t = j * PP_TILE + tid;
    const uint64_t w = t < N ? pp_weight(mind[(size_t)bh * N + t], kexp[bh]) : 0;
    uint64_t tt;
    const uint64_t ex = block_exscan_u64(w, s_w, &tt);
    if (ex <= local && local - ex < w) s_tok = t;
    __syncthreads();
    tok = s_tok >= 0 ? s_tok : (int)__umul64hi(word, (uint64_t)N);
  }
  const T* row = x + ((size_t)bh * N + tok) * D;
  for (int d = tid; d < D; d += PP_TILE) cent[((size_t)bh * C + c) * D + d] = to_f32(row[d]);
  if (tid == 0 && chosen) chosen[(size_t)bh * C + c] = tok;
}

struct PpPlan {
  int ntiles;
  size_t off_mind, off_tmax, off_tsum, off_k, total;
};

static PpPlan pp_plan(int B, int H, int N) {
  PpPlan p;
  const size_t BH = (size_t)B * H;
  p.ntiles = cdiv(N, PP_TILE);
  Carver cv(nullptr);
  p.off_mind = cv.used; cv.take<double>(BH * N);
  p.off_tmax = cv.used; cv.take<double>(BH * p.ntiles);
  p.off_tsum = cv.used; cv.take<uint64_t>(BH * p.ntiles);
  p.off_k = cv.used; cv.take<int>(BH);
  p.total = cv.used;
  return p;
}

template <typename T, int D>
static void pp_launch(const T* x, int BH, int N, int C, const uint64_t* words, float* cent, int32_t* chosen,
                      const PpPlan& p, char* w, hipStream_t stream) {
  double* mind = reinterpret_cast<double*>(w + p.off_mind);
  double* tmax = reinterpret_cast<double*>(w + p.off_tmax);
  uint64_t* tsum = reinterpret_cast<uint64_t*>(w + p.off_tsum);
  int* kexp = reinterpret_cast<int*>(w + p.off_k);
  const dim3 tiles(p.ntiles, BH);
  hipLaunchKernelGGL((pp_first_kernel<T, D>), dim3(BH), dim3(64), 0, stream, x, N, C, words, cent, chosen);
  if (C < 2) return;
  hipLaunchKernelGGL((pp_dist_kernel<T, D, true>), tiles, dim3(PP_TILE), 0, stream, x, N, C, 1, cent, mind, kexp,
                     tmax, tsum, p.ntiles);
  hipLaunchKernelGGL(pp_scale_kernel, dim3(BH), dim3(256), 0, stream, tmax, p.ntiles, N, kexp);
  hipLaunchKernelGGL(pp_weights_kernel, tiles, dim3(PP_TILE), 0, stream, mind, N, kexp, tsum, p.ntiles);
  for (int c = 1; c < C; ++c) {
    if (c > 1)
      hipLaunchKernelGGL((pp_dist_kernel<T, D, false>), tiles, dim3(PP_TILE), 0, stream, x, N, C, c, cent, mind,
                         kexp, tmax, tsum, p.ntiles);
    hipLaunchKernelGGL((pp_select_kernel<T, D>), dim3(BH), dim3(PP_TILE), 0, stream, x, N, C, c, words, mind, kexp,
                       tsum, p.ntiles, cent, chosen);
  }
}

}  // namespace svg

using namespace svg;

extern "C" size_t svgear_kmeanspp_workspace(int B, int H, int N, int D) {
  if (B < 1 || H < 1 || N < 1 || (D != 64 && D != 128)) return 0;
  return pp_plan(B, H, N).total;
}

extern "C" svgear_status svgear_kmeanspp(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                                         const uint64_t* words, float* centroids, int32_t* chosen, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  svgear_status st = check_common("kmeanspp", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (C < 1 || C > N || C > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "kmeanspp: C=%d must be in [1, min(N=%d, %d)]", C, N, SVGEAR_MAX_CLUSTERS);
  if (!x || !words || !centroids) return fail(SVGEAR_ERR_INVALID_ARG, "kmeanspp: null pointer");
  const PpPlan p = pp_plan(B, H, N);
  st = check_ws("kmeanspp", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  const int BH = B * H;
  if (dt == SVGEAR_BF16) {
    if (D == 128) pp_launch<bf16, 128>((const bf16*)x, BH, N, C, words, centroids, chosen, p, w, stream);
    else pp_launch<bf16, 64>((const bf16*)x, BH, N, C, words, centroids, chosen, p, w, stream);
  } else {
    if (D == 128) pp_launch<float, 128>((const float*)x, BH, N, C, words, centroids, chosen, p, w, stream);
    else pp_launch<float, 64>((const float*)x, BH, N, C, words, centroids, chosen, p, w, stream);
  }
  return check_launch("svgear_kmeanspp");
}
