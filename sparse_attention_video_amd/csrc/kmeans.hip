// k-means (Lloyd rounds), the cluster-contiguous permutation and the
// per-cluster means: svgear_kmeans and svgear_centroids.
//
// SVG2 summary, "Semantic-Aware Permutation via k-Means Clustering" (Q and K
// clustered independently per head; permute so each cluster is contiguous)
// and "Efficient System-Algorithm Co-Design" (centroid cache warm starts);
// SVG-EAR task page, walkthrough step 1 (k-means on the GPU returning the
// sorted order; a small kernel averaging each cluster in one pass).
//
// One Lloyd round is: prep (centroid MFMA operands) -> assign (MFMA distance
// tiles + exact refinement of near ties) -> tile histograms -> scan ->
// stable scatter (perm) -> chunked segment sums -> means.
#include <float.h>

#include <type_traits>

#include "common.h"
#include "host.h"
#include "scan.h"

namespace svg {

constexpr int KM_EXTRA = 16;        // extra K slots of the distance GEMM (norms, offset)
constexpr int KM_TOK_WG = 256;      // tokens per assign workgroup (4 waves x 64)
// candidate pruning of the tracking rounds pays from a few hundred centroids
// on (its bound matrix is C x C per head)
constexpr int KM_PRUNE_MIN_C = 256, KM_PRUNE_MAX_C = 1024;
constexpr int SORT_TILE = 4096;     // tokens per histogram / scatter tile
constexpr int MEAN_ROWS = 256;      // rows per segment-sum chunk
constexpr float PAD_NORM = 1e30f;   // squared norm given to padding centroids
constexpr int KM_PREP_ROWS = 32;    // centroid rows per prep workgroup
constexpr int KM_FULL_ROUNDS = 3;  // rounds whose update re-sorts every token
constexpr int KM_MSLOTS = 64;      // per-head counters (and sub-lists) the assign waves spread their atomics over
constexpr int KM_FX_BITS = 30;      // fixed-point values: |x| * 2^s < 2^30 (int32); sums of < 2^24 rows < 2^54

// --------------------------------------------------------------------------
// prep: per (batch, head), the bf16 operands of the distance GEMM, one row
// of KM_ROW(D) elements per centroid:
//   [0, D)          hi part of -2 c
//   [D, D + 16)     (1, 1, 1, n_hi, n_mid, n_lo, 0, ...)   n = ||c||^2 (fp32) split in three
//   [D + 16, 2D+16) lo part of -2 c
// Padding rows (c >= C) get zeros and n = PAD_NORM, so they never win.
// nmax[bh] collects the largest ||c||^2 (bit pattern) for the error window;
// it is cleared by km_scan_kernel or km_delta_kernel (and once before the
// first round).
// --------------------------------------------------------------------------
template <int D>
constexpr int km_row() { return 2 * D + KM_EXTRA; }

// Moved-token sub-list capacity: assign wave i of a head (64 tokens) appends
// to sub-list i mod KM_MSLOTS, so a sub-list never holds more than this.
inline __host__ __device__ int km_mcap(int N) {
  return ((N + KM_TOK_WG - 1) / KM_TOK_WG * 4 + KM_MSLOTS - 1) / KM_MSLOTS * 64;
}

template <int D>
__global__ void __launch_bounds__(256) km_prep_kernel(const float* __restrict__ cent, int C, int Cpad,
                                                      bf16* __restrict__ ops, uint32_t* __restrict__ nmax,
                                                      int32_t* __restrict__ mtot, float* __restrict__ cnorm) {
  constexpr int EPL = D / SV_WAVE;  // elements per lane
  constexpr int RW = km_row<D>();
  __shared__ double s_max[4];
  const int bh = blockIdx.y, lane = lane_id(), w = wave_id();
  const float* cb = cent + (size_t)bh * C * D;
  if (mtot && blockIdx.x == 0 && threadIdx.x < KM_MSLOTS) mtot[bh * KM_MSLOTS + threadIdx.x] = 0;  // read by the previous update
  double wmax = 0.0;
  // the wave's rows are loaded before the first one is processed
  constexpr int RR = KM_PREP_ROWS / 4;
  float vals[RR][EPL];
#pragma unroll
  for (int rr = 0; rr < RR; ++rr) {
    const int c = blockIdx.x * KM_PREP_ROWS + rr * 4 + w;
#pragma unroll
    for (int e = 0; e < EPL; ++e) vals[rr][e] = c < C ? cb[(size_t)c * D + lane + e * SV_WAVE] : 0.f;
  }
#pragma unroll
  for (int rr = 0; rr < RR; ++rr) {
    const int c = blockIdx.x * KM_PREP_ROWS + rr * 4 + w;
    if (c >= Cpad) break;
    bf16* row = ops + ((size_t)bh * Cpad + c) * RW;
    double cc = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane + e * SV_WAVE;
      const float v = vals[rr][e];
      bf16 hi, lo;
      split_bf16(-2.f * v, hi, lo);
      row[d] = hi;
      row[D + KM_EXTRA + d] = lo;
      cc += (double)v * (double)v;
    }
    cc = wave_sum_d(cc);
    if (c < C) wmax = fmax(wmax, cc);
    if (cnorm && lane == 0 && c < C) cnorm[(size_t)bh * Cpad + c] = (float)cc;  // ||c||^2 (fp64 sum, rounded once)
    if (lane < KM_EXTRA) {
      const float n = c < C ? (float)cc : PAD_NORM;
      const bf16 n_hi = (bf16)n;
      const float r1 = n - (float)n_hi;
      const bf16 n_mid = (bf16)r1;
      const bf16 n_lo = (bf16)(r1 - (float)n_mid);
      bf16 val = (bf16)0.f;
      if (lane < 3) val = (bf16)1.f;
      else if (lane == 3) val = n_hi;
      else if (lane == 4) val = c < C ? n_mid : (bf16)0.f;
      else if (lane == 5) val = c < C ? n_lo : (bf16)0.f;
      row[D + lane] = val;
    }
  }
  if (lane == 0) s_max[w] = wmax;
  __syncthreads();
  // the max of positive floats is the max of their bit patterns, so an
  // integer atomic max gives the same result in any order
  if (threadIdx.x == 0) {
    const double m = fmax(fmax(s_max[0], s_max[1]), fmax(s_max[2], s_max[3]));
    if (m > 0.0) atomicMax(&nmax[bh], __float_as_uint((float)(m * (1.0 + 1e-6))));
  }
}

// --------------------------------------------------------------------------
// Lower bounds on squared centroid distances, lb[a][c] <= ||c_a - c_c||^2, for
// the candidate pruning of the tracking rounds (Elkan's triangle-inequality
// bound: a centroid c with ||c_a - c_c|| > 2 ||x - c_a|| is strictly farther
// from x than c_a, so x's label cannot move to it).  A wave takes a 32 x 32
// tile from the hi parts of the prep operand rows (-2c rounded to bf16,
// within 2^-8 of each element): P = Ah.Ch estimates 4 c_a.c_c, and P / 2 is
// within 2^-7 (n_a + n_c) of 2 c_a.c_c (n = ||c||^2 from fp64 sums rounded
// once; fp32 sums of D products add below 1e-5), so lb = n_a + n_c - P / 2 -
// 0.02 (n_a + n_c).  The margin is loose, but the bound only has to fall
// below 4 R^2 where the exact distance does, and the squared distances of
// centroids lie far apart compared with it.
// --------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) km_cc_kernel(const bf16* __restrict__ ops, const float* __restrict__ cnorm,
                                                    int C, int Cpad, float* __restrict__ lb) {
  constexpr int RW = km_row<D>(), KS = D / 16;
  const int bh = blockIdx.y, lane = lane_id(), w = wave_id();
  const int nt = Cpad / 32, tile = blockIdx.x * 4 + w;
  if (tile >= nt * nt) return;
  const int a0 = (tile / nt) * 32, c0 = (tile % nt) * 32;
  const int half = lane >> 5, col = lane & 31;
  const bf16* ob = ops + (size_t)bh * Cpad * RW + 8 * half;
  const bf16* ra = ob + (size_t)(a0 + col) * RW;
  const bf16* rc = ob + (size_t)(c0 + col) * RW;
  bf16x8 ah[KS], ch[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    ah[ks] = *reinterpret_cast<const bf16x8*>(ra + 16 * ks);
    ch[ks] = *reinterpret_cast<const bf16x8*>(rc + 16 * ks);
  }
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(ah[ks], ch[ks], acc);
  // lane: column c = c0 + col, rows a = a0 + c_row(r, half)
  const float* nb = cnorm + (size_t)bh * Cpad;
  const int c = c0 + col;
  if (c >= C) return;
  const float nc = nb[c];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int a = a0 + c_row(r, half);
    if (a < C) {
      const float sn = nb[a] + nc;
      lb[((size_t)bh * C + a) * C + c] = sn - 0.5f * acc[r] - 0.02f * sn;
    }
  }
}

// --------------------------------------------------------------------------
// assign: label[n] = argmin_c ||x_n - c||^2 (ties to the lowest index).
//
// Each wave owns 64 tokens as two 32-token MFMA B tiles held in registers;
// the workgroup streams 32-centroid chunks of the prep operands through LDS.
// One 32x32 output tile is (centroid m, token n) ->
//   V = ||x||^2 + off + ||c||^2 - 2 x.c   (the extra K slots add the norms),
// an fp32 estimate of ||x - c||^2 + off with off >= 1 keeping it positive.
// The low `ib` bits of V's float pattern are replaced by the centroid index;
// the result orders like (V, index) and each lane keeps its 4 smallest with
// min/med3.  A rigorous bound W on the estimate's error (bf16 splitting of c
// and of fp32 x, fp32 accumulation, truncation of the low bits) decides:
//   key2 - key1 > W          -> label = index of key1 (provably the argmin)
//   else, <= 4 keys inside W -> exact fp64 distances of those candidates
//   else                     -> exact fp64 scan of every centroid
// The exact distances are summed by a fixed 64-lane butterfly.
// --------------------------------------------------------------------------
//
// PRUNE (tracking rounds, bf16): the workgroup takes 256 consecutive tokens of
// the order sorted by their current labels (perm), and only the centroids
// that can still be nearest to one of them: with R_a the largest distance
// of the workgroup's tokens of label a to c_a (an fp32 upper bound), c stays
// a candidate iff lb[a][c] <= 4 R_a^2 for some label a present; every other
// centroid is strictly farther from each such token than its c_a.  The list
// of candidates (ascending, in LDS) replaces 0 .. C-1: chunk rows are
// gathered from it and keys carry list positions, mapped back at the end.
template <typename T, int D, bool PRUNE = false, int CPT = 1>
__global__ void __launch_bounds__(256, sizeof(T) == 2 ? (D == 128 ? 3 : 2) : 1) km_assign_kernel(const T* __restrict__ x, const bf16* __restrict__ ops,
                                                        const uint32_t* __restrict__ nmax,
                                                        const float* __restrict__ cent, int N, int C, int Cpad, int ib,
                                                        int32_t* __restrict__ labels, int2* __restrict__ moved,
                                                        int32_t* __restrict__ mtot, uint32_t* __restrict__ r2max,
                                                        const int32_t* __restrict__ perm, const float* __restrict__ lb,
                                                        const int32_t* __restrict__ slab, int32_t* __restrict__ slab_new) {
  constexpr bool F32 = sizeof(T) == 4;
  static_assert(!(PRUNE && F32), "candidate pruning is built for bf16 tokens");
  constexpr int KS = D / 16;
  constexpr int RW = km_row<D>();          // operand row (bf16 elements)
  constexpr int SR = RW + 8;               // LDS row stride: an odd multiple of 16 bytes
  constexpr int U = RW / 8;                // 16-byte units per row
  constexpr int CHB = 32 * SR * 2;         // bytes of one staged chunk in LDS
  constexpr int NJ = (CHB + 1023) / 1024;  // 1 KB direct-to-LDS loads per chunk
  constexpr int NJW = (NJ + 3) / 4;        // per wave (load j = 4 k + wave)
  __shared__ __attribute__((aligned(1024))) bf16 s_ops[2][NJ * 512];

  const int bh = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int half = lane >> 5, col = lane & 31;
  const T* xb = x + (size_t)bh * N * D;
  const bf16* ob = ops + (size_t)bh * Cpad * RW;
  const float* cb = cent + (size_t)bh * C * D;
  const int tok0 = blockIdx.x * KM_TOK_WG + w * 64;
  const float u = 5.9604645e-08f;  // 2^-24

  bf16x8 bx[2][KS];
  bf16x8 bxl[2][F32 ? KS : 1];
  bf16x8 bext[2];
  float xx[2];
  int lold[2];  // previous labels (tracking rounds), loaded with the rows
  int tokn[2];  // token index of this lane's column of tile t (N: none)
  // chunk staging straight from global memory into LDS (no registers): a
  // chunk is 32 contiguous operand rows in global memory and 32 rows of
  // stride SR in LDS.  Load j fills LDS bytes [1024 j, 1024 j + 1024) of the
  // buffer, lane L the 16 bytes at o = 1024 j + 16 L: byte o % (2 SR) of row
  // o / (2 SR).  Pad bytes (never read) take the chunk's first 16 bytes.
  // The buffer form keeps the LDS-read waits of the products partial.
  uint32_t goff[NJW];
#pragma unroll
  for (int k = 0; k < NJW; ++k) {
    const int o = 1024 * (4 * k + w) + 16 * lane;
    const int r = o / (2 * SR), cb = o - r * (2 * SR);
    goff[k] = (o < CHB && cb < 2 * RW) ? (uint32_t)(r * 2 * RW + cb) : 0u;
  }
  const __amdgpu_buffer_rsrc_t rops =
      __builtin_amdgcn_make_buffer_rsrc((void*)ob, (short)0, Cpad * RW * 2, 0x00020000);
  // the largest centroid norm bound of the error window, read up front
  const uint32_t nmax_bits = nmax[bh];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int pos = tok0 + 32 * t + col;
    tokn[t] = pos < N ? (PRUNE ? perm[(size_t)bh * N + pos] : pos) : N;
  }
  // previous labels (tracking rounds; PRUNE: by position in the sorted
  // order), read unconditionally so that every path issues the same loads
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool ok = tokn[t] < N;
    if constexpr (PRUNE) {
      const int v = slab[(size_t)bh * N + min(tok0 + 32 * t + col, N - 1)];
      lold[t] = ok ? v : -1;
    } else {
      const int v = labels[(size_t)bh * N + min(tokn[t], N - 1)];
      lold[t] = (moved && ok && half == 0) ? v : -1;
    }
  }
  if constexpr (!F32) {
    // both tiles' rows are in flight before either is used (one memory
    // latency, not two); a column past N reads row N - 1, whose results the
    // kernel never stores (labels, moves and bounds skip such columns)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const size_t nr = (size_t)min(tokn[t], N - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bx[t][ks] = *reinterpret_cast<const bf16x8*>(xb + nr * D + 16 * ks + 8 * half);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = tokn[t];
    const bool ok = n < N;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 16 * ks + 8 * half;
      if constexpr (!F32) {
        const bf16x8 v = bx[t][ks];
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)v[e] * (float)v[e];
      } else {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
        if (ok) {
          f32x4 a = *reinterpret_cast<const f32x4*>(xb + (size_t)n * D + d0);
          f32x4 b = *reinterpret_cast<const f32x4*>(xb + (size_t)n * D + d0 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[e + 4] = b[e]; }
        }
        bf16x8 h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 hh, ll;
          split_bf16(f[e], hh, ll);
          h[e] = hh;
          l[e] = ll;
          part += f[e] * f[e];
        }
        bx[t][ks] = h;
        bxl[t][ks % (F32 ? KS : 1)] = l;
      }
    }
    xx[t] = part + shfl_xor(part, 32);
  }
  if (r2max) {
    // an upper bound on max ||x||^2 (fp32 sum of D squares, relative error
    // below D u < 1e-5), the basis of the fixed-point scale
    float m = fmaxf(xx[0], xx[1]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, SV_WAVE));
    if (lane == 0 && m > 0.f)
      atomicMax(&r2max[bh * KM_MSLOTS + ((blockIdx.x * 4 + w) & (KM_MSLOTS - 1))], __float_as_uint(m * (1.f + 1e-5f)));
  }

  const uint32_t imask = (1u << ib) - 1u;
  float key[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) key[t][k] = FLT_MAX;

  // candidate list (PRUNE): positions 0 .. nlist-1 hold centroid indices
  // (chunk 0 reserves 32 positions for the own labels, so a list holds up
  // to C + 31 positions; the caller's ib covers them)
  __shared__ int s_cand[PRUNE ? 256 * CPT + 32 : 1];
  __shared__ uint32_t s_r2[PRUNE ? KM_TOK_WG : 1];
  __shared__ int s_pos[PRUNE ? 64 : 1];
  __shared__ int s_cnt[4];
  __shared__ int s_cnt4[PRUNE ? CPT : 1][4];
  int nlist = C, nfirst = 0, a_lo = 0, a_hi = 0;
  if constexpr (PRUNE) {
    // labels of the workgroup's tokens span a_lo .. a_hi (sorted order)
    const int p0 = blockIdx.x * KM_TOK_WG, p1 = min(N, p0 + KM_TOK_WG) - 1;
    a_lo = slab[(size_t)bh * N + p0];
    a_hi = slab[(size_t)bh * N + p1];
    const bool narrow = a_hi - a_lo < 64;
    s_r2[tid] = 0u;
    __syncthreads();
    if (narrow && half == 0)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (tokn[t] < N) s_r2[lold[t] - a_lo] = 1u;  // present labels
    __syncthreads();
    if (narrow && w == 0) {
      // chunk 0 = the present labels, ascending; s_pos: label -> position
      const bool pres = s_r2[lane] != 0u;
      const uint64_t bal = ballot(pres);
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (pres) s_cand[pos] = a_lo + lane;
      s_pos[lane] = pos;
      if (lane == 0) s_cnt[0] = __popcll(bal);
    }
    __syncthreads();
    const int k = narrow ? s_cnt[0] : 33;
    if (k <= 32) {
      nfirst = k;
      nlist = 32;  // chunk 0 for now; the other candidates follow its products
      for (int q = k + tid; q < 32; q += 256) s_cand[q] = s_cand[0];
    } else {
      // no pruning for this workgroup: every centroid, in order
      for (int c = tid; c < C; c += 256) s_cand[c] = c;
      for (int q = C + tid; q < ((C + 31) & ~31); q += 256) s_cand[q] = s_cand[0];
    }
    __syncthreads();
  }
  // PRUNE: the bound rows of the first four own labels are read now, so their
  // latency overlaps chunk 0's staging (the staging wait covers them too)
  float lv0[4][PRUNE ? CPT : 1];
  if constexpr (PRUNE) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float* row = lb + ((size_t)bh * C + s_cand[jj < nfirst ? jj : 0]) * C;
#pragma unroll
      for (int u = 0; u < CPT; ++u) lv0[jj][u] = row[min(tid + 256 * u, C - 1)];
    }
  }
  auto stage = [&](int c0, int buf) {
#pragma unroll
    for (int k = 0; k < NJW; ++k)
      if (4 * k + w < NJ) {
        uint32_t go = goff[k];
        int so = c0 * RW * 2;
        if constexpr (PRUNE) {
          // row r of the chunk is candidate c0 + r (pad bytes: its row start)
          const int o = 1024 * (4 * k + w) + 16 * lane;
          const int r = min(o / (2 * SR), 31), cb2 = o - r * (2 * SR);
          go = (uint32_t)s_cand[c0 + r] * (uint32_t)(RW * 2) + (uint32_t)((o < CHB && cb2 < 2 * RW) ? cb2 : 0);
          so = 0;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rops, (__attribute__((address_space(3))) void*)(&s_ops[buf][512 * (4 * k + w)]), 16, (int)go, so, 0, 0);
      }
  };
  // this wave's staging loads have landed (vector-memory count 0; the export
  // and LDS counts left at their maxima)
  auto staged = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

  // extra K slots of the token side: (||x||^2 hi, lo, offset, 1, 1, 1)
  // the offset keeps V positive; it is set from a first window estimate below
  const float s_split = F32 ? 3.01f : 1.0f;
  const int kprod = D * (F32 ? 3 : 2) + KM_EXTRA;
  const float gam = (kprod * u) / (1.f - kprod * u);
  stage(0, 0);
  staged();
  __syncthreads();
  const float cm_pre = sqrtf(__uint_as_float(nmax_bits)) * (1.f + 1e-5f);
  float E0[2], off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float X = sqrtf(xx[t]) * (1.f + 1e-6f);
    const float xxb = xx[t] * (1.f + 2e-5f) + 1e-30f;
    const float cm = cm_pre;
    const float pre_ = u * cm * cm + 4.f * s_split * 3.8146973e-06f * X * cm;  // 2^-18
    const float e0 = 1.25f * (pre_ + gam * (xxb + 2.f + cm * cm + 2.05f * X * cm));
    const float o = 1.f + 4.f * e0 + 4e-5f * xxb;
    E0[t] = 1.25f * (pre_ + gam * (xxb + o + 2.f + cm * cm + 2.05f * X * cm));
    off[t] = o;
    bf16x8 ex = {};
    if (half == 0) {
      bf16 xh, xl;
      split_bf16(xx[t], xh, xl);
      ex[0] = xh;
      ex[1] = xl;
      ex[2] = (bf16)o;
      ex[3] = (bf16)1.f;
      ex[4] = (bf16)1.f;
      ex[5] = (bf16)1.f;
    }
    bext[t] = ex;
  }
  const float q = ldexpf(1.f, ib - 23);

  // step i of the 2 KS + 1 products: the extra slots (i = 0), the hi part of
  // -2c (1 .. KS), the lo part (KS + 1 .. 2 KS); each step's centroid
  // fragment is read two steps ahead (LDS latency exceeds one step's products)
  constexpr int NSTEP = 2 * KS + 1;
  auto frag_off = [&](int i) {
    return (i == 0 ? D : i <= KS ? 16 * (i - 1) : D + KM_EXTRA + 16 * (i - 1 - KS)) + 8 * half;
  };
  auto mma = [&](int buf, f32x16& acc0, f32x16& acc1) {
    const bf16* R = &s_ops[buf][col * SR];
    acc0 = f32x16{};
    acc1 = f32x16{};
    bf16x8 fr[3];
    fr[0] = *reinterpret_cast<const bf16x8*>(R + frag_off(0));
    fr[1] = *reinterpret_cast<const bf16x8*>(R + frag_off(1));
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + 2 < NSTEP) fr[(i + 2) % 3] = *reinterpret_cast<const bf16x8*>(R + frag_off(i + 2));
      const bf16x8 a = fr[i % 3];
      if (i == 0) {
        acc0 = mfma_bf16(a, bext[0], acc0);
        acc1 = mfma_bf16(a, bext[1], acc1);
      } else {
        const int ks = (i - 1) % KS;
        acc0 = mfma_bf16(a, bx[0][ks], acc0);
        acc1 = mfma_bf16(a, bx[1][ks], acc1);
        if (F32 && i <= KS) {
          acc0 = mfma_bf16(a, bxl[0][ks % (F32 ? KS : 1)], acc0);
          acc1 = mfma_bf16(a, bxl[1][ks % (F32 ? KS : 1)], acc1);
        }
      }
    }
    // pin the read-ahead (mask bits: 0x100 LDS read, 0x008 MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + 2 < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (F32 && i >= 1 && i <= KS)
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };
  // keys: the low ib bits of V's pattern carry the centroid index; keep the
  // 4 smallest per lane with med3 and an integer min (keys are positive floats,
  // whose order is the order of their bit patterns)
  auto keys = [&](int c0, const f32x16& acc0, const f32x16& acc1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t idx = (uint32_t)(c0 + c_row(r, half));
      const float k0 = __uint_as_float((__float_as_uint(acc0[r]) & ~imask) | idx);
      const float k1 = __uint_as_float((__float_as_uint(acc1[r]) & ~imask) | idx);
      key[0][3] = med3f(key[0][2], key[0][3], k0);
      key[0][2] = med3f(key[0][1], key[0][2], k0);
      key[0][1] = med3f(key[0][0], key[0][1], k0);
      key[0][0] = minkey(key[0][0], k0);
      key[1][3] = med3f(key[1][2], key[1][3], k1);
      key[1][2] = med3f(key[1][1], key[1][2], k1);
      key[1][1] = med3f(key[1][0], key[1][1], k1);
      key[1][0] = minkey(key[1][0], k1);
    }
  };
  // PRUNE: only keys within the tie window of a token's final best key k are
  // ever used (the label, the refinement candidates, their count).  With kb
  // the token's best key so far (both halves), k <= kb, and the window
  // W(k) = 2 E0 + 2.5 q (2 k + 2 E0 + 1) grows with k, so an estimate V >
  // thr = (kb + W(kb)) (1 + 4 q) gives a key (V with its low ib bits replaced,
  // > V (1 - q)) above k + W(k) with room for the fp32 roundings: it cannot
  // enter the window.  A tile whose 16 estimates lie above thr in every lane
  // of the wave leaves the windowed part of the lists unchanged, and after
  // chunk 0 (the own labels) that is the common case, so its insertion is
  // skipped.
  float thr[2] = {INFINITY, INFINITY};
  auto set_thr = [&](int t) {
    const float kb = fminf(key[t][0], shfl_xor(key[t][0], 32));
    const float W = 2.f * E0[t] + q * (2.f * kb + 2.f * E0[t] + 1.f) * 2.5f;
    thr[t] = (kb + W) * (1.f + 4.f * q);
  };
  auto keys_win = [&](int c0, const f32x16& acc0, const f32x16& acc1) {
    float m0 = acc0[0], m1 = acc1[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      m0 = fminf(m0, acc0[r]);
      m1 = fminf(m1, acc1[r]);
    }
    if (ballot(m0 <= thr[0])) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t idx = (uint32_t)(c0 + c_row(r, half));
        const float k0 = __uint_as_float((__float_as_uint(acc0[r]) & ~imask) | idx);
        key[0][3] = med3f(key[0][2], key[0][3], k0);
        key[0][2] = med3f(key[0][1], key[0][2], k0);
        key[0][1] = med3f(key[0][0], key[0][1], k0);
        key[0][0] = minkey(key[0][0], k0);
      }
      set_thr(0);
    }
    if (ballot(m1 <= thr[1])) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t idx = (uint32_t)(c0 + c_row(r, half));
        const float k1 = __uint_as_float((__float_as_uint(acc1[r]) & ~imask) | idx);
        key[1][3] = med3f(key[1][2], key[1][3], k1);
        key[1][2] = med3f(key[1][1], key[1][2], k1);
        key[1][1] = med3f(key[1][0], key[1][1], k1);
        key[1][0] = minkey(key[1][0], k1);
      }
      set_thr(1);
    }
  };
  int ci0 = 0;
  if constexpr (PRUNE) {
    if (nfirst > 0) {
      // chunk 0 holds the workgroup's own labels: each token's estimate V of
      // ||x - c_a||^2 + off (a in chunk 0) bounds its distance to its own
      // centroid, ||x - c_a||^2 <= V - off + 2 E0 (+ the rounding of ||x||^2
      // and its split, below 3e-5 ||x||^2)
      f32x16 acc0, acc1;
      mma(0, acc0, acc1);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x16& acc = t ? acc1 : acc0;
        const int p = tokn[t] < N ? s_pos[lold[t] - a_lo] : 0;
        const int hp = (p >> 2) & 1, rs = ((p >> 3) << 2) | (p & 3);
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) v = r == rs ? acc[r] : v;
        const float vo = shfl_xor(v, 32);
        const float V = half == hp ? v : vo;
        const float offb = (float)(bf16)off[t];
        const float u2 = fmaxf(0.f, V - offb + 2.f * E0[t] + 3e-5f * xx[t]) * (1.f + 1e-5f);
        // (bit pattern + 1: present labels stay nonzero even at distance 0)
        if (half == 0 && tokn[t] < N) atomicMax(&s_r2[lold[t] - a_lo], __float_as_uint(u2) + 1u);
      }
      __syncthreads();
      // the other candidates, ascending, from position 32: thread tid tests
      // centroids tid + 256 u against the own labels, 4 labels' bound loads
      // in flight at a time
      bool keep[CPT];
#pragma unroll
      for (int u = 0; u < CPT; ++u) keep[u] = false;
      for (int i0 = 0; i0 < nfirst; i0 += 4) {
        float thr[4];
        const float* lrow[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int a = s_cand[i0 + jj < nfirst ? i0 + jj : 0];
          thr[jj] = i0 + jj < nfirst ? 4.f * __uint_as_float(s_r2[a - a_lo] - 1u) * (1.f + 3e-5f) : -1.f;
          lrow[jj] = lb + ((size_t)bh * C + a) * C;
        }
        float lv[4][CPT];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int u = 0; u < CPT; ++u) lv[jj][u] = i0 == 0 ? lv0[jj][u] : lrow[jj][min(tid + 256 * u, C - 1)];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int u = 0; u < CPT; ++u) keep[u] = keep[u] || lv[jj][u] <= thr[jj];
      }
      uint64_t bal[CPT];
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = tid + 256 * u;
        // (the own labels are already in chunk 0)
        keep[u] = keep[u] && c < C && !(c >= a_lo && c <= a_hi && s_r2[c - a_lo] != 0u);
        bal[u] = ballot(keep[u]);
        if (lane == 0) s_cnt4[u][w] = __popcll(bal[u]);
      }
      __syncthreads();
      int base = 32;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        int o = base;
        for (int v = 0; v < w; ++v) o += s_cnt4[u][v];
        if (keep[u])
          s_cand[o + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u], 0))] =
              tid + 256 * u;
        base += s_cnt4[u][0] + s_cnt4[u][1] + s_cnt4[u][2] + s_cnt4[u][3];
      }
      nlist = base;
      for (int q = nlist + tid; q < ((nlist + 31) & ~31); q += 256) s_cand[q] = s_cand[0];
      __syncthreads();
      if (nlist > 32) stage(32, 1);
      // chunk 0's keys; its positions past the own labels are padding
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (c_row(r, half) >= nfirst) {
          acc0[r] = FLT_MAX;
          acc1[r] = FLT_MAX;
        }
      keys(0, acc0, acc1);
      set_thr(0);
      set_thr(1);
      if (nlist > 32) staged();
      __syncthreads();
      ci0 = 1;
    }
  }
  const int nchunk = PRUNE ? (nlist + 31) / 32 : Cpad / 32;
  for (int ci = ci0; ci < nchunk; ++ci) {
    const int buf = ci & 1;
    const bool more = ci + 1 < nchunk;
    if (more) stage((ci + 1) * 32, buf ^ 1);
    f32x16 acc0, acc1;
    mma(buf, acc0, acc1);
    if (PRUNE && ci * 32 + 32 > nlist) [[unlikely]] {
      // list positions past the last candidate (padding) never enter a list
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (ci * 32 + c_row(r, half) >= nlist) {
          acc0[r] = FLT_MAX;
          acc1[r] = FLT_MAX;
        }
    }
    if constexpr (PRUNE)
      keys_win(ci * 32, acc0, acc1);
    else
      keys(ci * 32, acc0, acc1);
    if (more) staged();
    __syncthreads();
  }

  // merge the two halves' lists (they hold different centroids of the same tokens)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = shfl_xor(key[t][k], 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float kk = o[k];
      key[t][3] = med3f(key[t][2], key[t][3], kk);
      key[t][2] = med3f(key[t][1], key[t][2], kk);
      key[t][1] = med3f(key[t][0], key[t][1], kk);
      key[t][0] = minkey(key[t][0], kk);
    }
  }

  int lab[2], ncand[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float k1v = key[t][0];
    const float W = 2.f * E0[t] + q * (2.f * k1v + 2.f * E0[t] + 1.f) * 2.5f;
    lab[t] = (int)(__float_as_uint(k1v) & imask);
    if constexpr (PRUNE) lab[t] = s_cand[min(lab[t], nlist - 1)];  // list position -> centroid
    int nc = 1;
#pragma unroll
    for (int k = 1; k < 4; ++k) nc += (key[t][k] - k1v <= W) ? 1 : 0;
    ncand[t] = nc;  // 1: decided; 2..3: refine candidates; 4: full scan
  }

  // Near ties: exact distances of the candidates, one flagged token at a time.
  // 2-3 candidates: each 16-lane row of the wave evaluates one centroid (a lane
  // takes D/16 coordinates, fp32, then a fixed 16-lane butterfly: pairwise
  // summation, error <= (log2 D + 3) u D, far inside the 1e-5 relative tie
  // tolerance).  4 keys inside the window (rare): every centroid is scanned,
  // one per lane, with fp64 sums and a wave argmin.
  constexpr int EPG = D / 16;
  const int grp = lane >> 4, gl = lane & 15;
  __shared__ float s_x[4][D];
  // tokens whose label changes (tracking rounds only): (token, old | new << 16)
  int2 mv[2];
  uint64_t mvb[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n_mine = tokn[t];
    uint64_t todo = ballot(half == 0 && n_mine < N && ncand[t] > 1);
    while (todo) {
      const int src = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int n = __shfl(n_mine, src, SV_WAVE);
      const int nc = __shfl(ncand[t], src, SV_WAVE);
      float best = 0.f;
      int bidx = -1;
      if (nc < 4) {
        float xv[EPG];
#pragma unroll
        for (int e = 0; e < EPG; ++e) xv[e] = to_f32(xb[(size_t)n * D + gl * EPG + e]);
        // every lane needs all three candidates of lane src (a shuffle returns the
        // source lane's register, so each key is fetched on its own)
        const uint32_t c0 = __float_as_uint(__shfl(key[t][0], src, SV_WAVE)) & imask;
        const uint32_t c1 = __float_as_uint(__shfl(key[t][1], src, SV_WAVE)) & imask;
        const uint32_t c2 = __float_as_uint(__shfl(key[t][2], src, SV_WAVE)) & imask;
        int c = (int)(grp == 0 ? c0 : grp == 1 ? c1 : c2);
        const bool live = grp < nc && c < (PRUNE ? nlist : C);
        if (!live) c = 0;
        if constexpr (PRUNE) c = s_cand[c];  // list position -> centroid
        const float* cr = cb + (size_t)c * D + gl * EPG;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPG; ++e) {
          const float dv = xv[e] - cr[e];
          part = fmaf(dv, dv, part);
        }
        const float dist = row16_sum(part);
#pragma unroll
        for (int g = 0; g < 3; ++g) {
          const float dg = __shfl(dist, 16 * g, SV_WAVE);
          const int cg = __shfl(c, 16 * g, SV_WAVE);
          const bool lg = __shfl((int)live, 16 * g, SV_WAVE) != 0;
          if (lg && (bidx < 0 || dg < best || (dg == best && cg < bidx))) {
            best = dg;
            bidx = cg;
          }
        }
      } else {
        for (int d = lane; d < D; d += SV_WAVE) s_x[w][d] = to_f32(xb[(size_t)n * D + d]);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        double bd = 0.0;
        int bi = -1;
        for (int c = lane; c < C; c += SV_WAVE) {
          const float* cr = cb + (size_t)c * D;
          double acc = 0.0;
          for (int d = 0; d < D; d += 4) {
            const f32x4 cv = *reinterpret_cast<const f32x4*>(cr + d);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double dv = (double)s_x[w][d + e] - (double)cv[e];
              acc = fma(dv, dv, acc);
            }
          }
          if (bi < 0 || acc < bd) { bd = acc; bi = c; }  // c ascends within a lane
        }
        // wave argmin of (distance, index)
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const double od = shfl_xor_d(bd, m);
          const int oi = __shfl_xor(bi, m, SV_WAVE);
          if (oi >= 0 && (bi < 0 || od < bd || (od == bd && oi < bi))) { bd = od; bi = oi; }
        }
        bidx = bi;
        __builtin_amdgcn_wave_barrier();
      }
      if (lane == src) lab[t] = bidx;
    }
    const bool mine = half == 0 && n_mine < N;
    const int lnew = min(lab[t], C - 1);
    if (moved) {
      const int lo = mine ? lold[t] : lnew;
      mvb[t] = ballot(lo != lnew);
      mv[t] = make_int2(n_mine, lo | (lnew << 16));
    }
    if (mine) {
      if constexpr (PRUNE)
        slab_new[(size_t)bh * N + tok0 + 32 * t + col] = lnew;  // by position (the sorted order)
      else
        labels[(size_t)bh * N + n_mine] = lnew;
    }
  }
  if (moved) {
    // one reservation per wave in its sub-list; the order of the list is
    // immaterial (the update adds integers)
    const int n0 = __popcll(mvb[0]), nt = n0 + __popcll(mvb[1]);
    if (nt > 0) {
      const int sl = (blockIdx.x * 4 + w) & (KM_MSLOTS - 1), cap = km_mcap(N);
      int base = 0;
      if (lane == 0) base = atomicAdd(&mtot[bh * KM_MSLOTS + sl], nt);
      base = __shfl(base, 0, SV_WAVE);
      int2* mb = moved + ((size_t)bh * KM_MSLOTS + sl) * cap;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if ((mvb[t] >> lane) & 1) {
          const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mvb[t] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mvb[t], 0));
          mb[base + (t ? n0 : 0) + r] = mv[t];
        }
    }
  }
}

// --------------------------------------------------------------------------
// tile histograms: counts[bh][tile][c] = #tokens of tile with label c
// --------------------------------------------------------------------------
__global__ void km_clear_kernel(uint32_t* __restrict__ v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v[i] = 0u;
}

__global__ void __launch_bounds__(256) km_hist_kernel(const int32_t* __restrict__ labels, int N, int C, int ntiles,
                                                      int32_t* __restrict__ counts) {
  __shared__ int32_t h[SVGEAR_MAX_CLUSTERS];
  const int bh = blockIdx.y, tile = blockIdx.x;
  for (int c = threadIdx.x; c < C; c += 256) h[c] = 0;
  __syncthreads();
  const int n0 = tile * SORT_TILE, n1 = min(N, n0 + SORT_TILE);
  const int32_t* lb = labels + (size_t)bh * N;
  // all of a thread's labels are loaded before the first count
  constexpr int PER = SORT_TILE / 256;
  int lab[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = n0 + threadIdx.x + 256 * i;
    lab[i] = n < n1 ? lb[n] : -1;
  }
  // a wave's 64 labels of a step are consecutive tokens: each run of equal
  // labels adds its length once (labels grouped by value give few runs)
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int l = lab[i];
    const int prev = __shfl_up(l, 1, SV_WAVE);
    const bool head = lane == 0 || prev != l;
    const uint64_t heads = ballot(head);
    const uint64_t later = heads & ~((2ull << lane) - 1ull);  // (lane 63: 2 << 63 wraps to 0)
    const int len = (lane == 63 || later == 0ull ? 64 : __builtin_ctzll(later)) - lane;
    if (head && l >= 0) atomicAdd(&h[l], len);
  }
  __syncthreads();
  int32_t* cnt = counts + ((size_t)bh * ntiles + tile) * C;
  for (int c = threadIdx.x; c < C; c += 256) cnt[c] = h[c];
}

// --------------------------------------------------------------------------
// scan: offsets (cluster starts), per-tile bases (in place over counts) and
// the segment-sum chunk list.  One block of 1024 threads per (batch, head).
// --------------------------------------------------------------------------
constexpr int KM_SCAN_LDS = 16384;  // tile histograms of a head held in LDS (64 KB)

__global__ void __launch_bounds__(1024) km_scan_kernel(int32_t* __restrict__ counts, int N, int C, int ntiles,
                                                       int rows, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ chunk_start, uint32_t* __restrict__ nmax) {
  __shared__ int sm[16];
  __shared__ int s_cnt[KM_SCAN_LDS];
  const int bh = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) nmax[bh] = 0u;  // the assign kernel of this round has finished
  int32_t* cnt = counts + (size_t)bh * ntiles * C;
  const int M = ntiles * C;
  const bool in_lds = M <= KM_SCAN_LDS;
  if (in_lds) {
    // the whole [ntiles][C] block with coalesced loads, all in flight together
    constexpr int PER = KM_SCAN_LDS / 1024;
    int v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 1024 * k;
      v[k] = i < M ? cnt[i] : 0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 1024 * k;
      if (i < M) s_cnt[i] = v[k];
    }
    __syncthreads();
  }
  // the tile loops load SB tiles of all 4 clusters before using any, so the
  // loads are in flight together rather than one latency each
  constexpr int SB = 8;
  int tot[4] = {0, 0, 0, 0}, nch[4];
  int sum = 0, csum = 0;
  if (in_lds) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = tid * 4 + e;
      if (c < C)
        for (int t = 0; t < ntiles; ++t) tot[e] += s_cnt[t * C + c];
    }
  } else {
    for (int t0 = 0; t0 < ntiles; t0 += SB) {
      int v[4][SB];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int c = tid * 4 + e;
          v[e][i] = (c < C && t0 + i < ntiles) ? cnt[(size_t)(t0 + i) * C + c] : 0;
        }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < SB; ++i) tot[e] += v[e][i];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    nch[e] = (tot[e] + rows - 1) / rows;
    sum += tot[e];
    csum += nch[e];
  }
  int total, ctotal;
  int base = block_exscan(sum, sm, &total);
  int cbase = block_exscan(csum, sm, &ctotal);
  int32_t* off = offsets + (size_t)bh * (C + 1);
  int32_t* cs = chunk_start + (size_t)bh * (C + 1);
  int b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = tid * 4 + e;
    if (c < C) {
      off[c] = base;
      cs[c] = cbase;
    }
    b[e] = base;
    base += tot[e];
    cbase += nch[e];
  }
  if (in_lds) {
    // per-tile bases in place, then one coalesced write of the block
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = tid * 4 + e;
      if (c < C)
        for (int t = 0; t < ntiles; ++t) {
          const int v = s_cnt[t * C + c];
          s_cnt[t * C + c] = b[e];
          b[e] += v;
        }
    }
    __syncthreads();
    for (int i = tid; i < M; i += 1024) cnt[i] = s_cnt[i];
  } else {
    for (int t0 = 0; t0 < ntiles; t0 += SB) {
      int v[4][SB];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int c = tid * 4 + e;
          v[e][i] = (c < C && t0 + i < ntiles) ? cnt[(size_t)(t0 + i) * C + c] : 0;
        }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int c = tid * 4 + e;
          if (c < C && t0 + i < ntiles) cnt[(size_t)(t0 + i) * C + c] = b[e];
          b[e] += v[e][i];
        }
    }
  }
  if (tid == 0) {
    off[C] = total;
    cs[C] = ctotal;
  }
}

// --------------------------------------------------------------------------
// stable scatter: perm[dest] = token, tokens of one cluster in original order.
// Each wave owns a contiguous quarter of the tile; equal labels inside a
// 64-token step are matched with ballots over the label bits, so ranks come
// out in lane order with no atomics.  The tile is first ordered by cluster in
// LDS and then written out in that order, so neighbouring lanes store to
// neighbouring addresses of perm (one run per cluster) instead of scattering
// every token on its own.
// --------------------------------------------------------------------------
constexpr int KM_SCATTER_CPT = SVGEAR_MAX_CLUSTERS / 256;  // clusters per thread in the tile scan

inline size_t km_scatter_lds(int C) { return (size_t)(5 * C + 3 * SORT_TILE) * sizeof(int32_t); }

// With src_map, perm gets src_map[n] instead of n (regrouping a permuted
// order: n is then a position of it); with slab_out, the labels in the new
// order as well.
__global__ void __launch_bounds__(256) km_scatter_kernel(const int32_t* __restrict__ labels,
                                                         const int32_t* __restrict__ tile_base, int N, int C,
                                                         int ntiles, int ib, int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ src_map,
                                                         int32_t* __restrict__ slab_out) {
  // [4][C] per-wave bases inside the tile | [C] tile position -> perm index
  // shift per cluster | [SORT_TILE] tokens and [SORT_TILE] destinations in
  // cluster order
  extern __shared__ int32_t hw[];
  __shared__ int s_scan[16];
  int32_t* shift = hw + 4 * C;
  int32_t* s_tok = shift + C;
  int32_t* s_dst = s_tok + SORT_TILE;
  int32_t* s_lab = s_dst + SORT_TILE;
  const int bh = blockIdx.y, tile = blockIdx.x, lane = lane_id(), w = wave_id();
  const int32_t* lb = labels + (size_t)bh * N;
  int32_t* pb = perm + (size_t)bh * N;
  for (int c = threadIdx.x; c < 4 * C; c += 256) hw[c] = 0;
  // each thread scans a contiguous run of clusters; its tile bases are
  // loaded now and used after the counting pass
  const int per = (C + 255) / 256, cr = threadIdx.x * per;
  const int32_t* tb = tile_base + ((size_t)bh * ntiles + tile) * C;
  int tbv[KM_SCATTER_CPT];
#pragma unroll
  for (int j = 0; j < KM_SCATTER_CPT; ++j) tbv[j] = (j < per && cr + j < C) ? tb[cr + j] : 0;
  __syncthreads();
  const int q0 = tile * SORT_TILE + w * (SORT_TILE / 4);
  const int q1 = min(N, q0 + SORT_TILE / 4);
  int32_t* mine = hw + w * C;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the wave's labels are loaded once, before either pass
  constexpr int STEPS = SORT_TILE / 4 / SV_WAVE;
  int labv[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int n = q0 + i * SV_WAVE + lane;
    labv[i] = n < q1 ? lb[n] : 0;
  }
  // counting pass: the rank of each token among the equal labels of its
  // step (bits 0-7) and their count (bits 8-15) are kept for the placing
  // pass; the lowest such lane (rank 0) adds the count
  int rk[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int n0 = q0 + i * SV_WAVE;
    if (n0 >= q1) break;
    const bool ok = n0 + lane < q1;
    const int lab = labv[i];
    uint64_t peers = ballot(ok);
    for (int b = 0; b < ib; ++b) {
      const bool bit = (lab >> b) & 1;
      const uint64_t m = ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt), cnt = __popcll(peers);
    rk[i] = rank | (cnt << 8);
    if (ok && rank == 0) mine[lab] += cnt;
  }
  // tile position of each (wave, cluster) run: clusters in order, waves in
  // order inside a cluster
  __syncthreads();
  {
    int sum = 0;
#pragma unroll
    for (int j = 0; j < KM_SCATTER_CPT; ++j) {
      const int c = cr + j;
      if (j < per && c < C) sum += hw[c] + hw[C + c] + hw[2 * C + c] + hw[3 * C + c];
    }
    int total;
    int base = block_exscan(sum, s_scan, &total);
#pragma unroll
    for (int j = 0; j < KM_SCATTER_CPT; ++j) {
      const int c = cr + j;
      if (j < per && c < C) {
        shift[c] = tbv[j] - base;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const int v = hw[ww * C + c];
          hw[ww * C + c] = base;
          base += v;
        }
      }
    }
  }
  __syncthreads();
  // placing pass: tokens and their perm indices in cluster order
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int n0 = q0 + i * SV_WAVE;
    if (n0 >= q1) break;
    const int n = n0 + lane;
    if (n < q1) {
      const int lab = labv[i], rank = rk[i] & 255;
      const int pos = mine[lab] + rank;
      s_tok[pos] = n;
      s_dst[pos] = pos + shift[lab];
      s_lab[pos] = lab;
      if (rank == 0) mine[lab] = pos + (rk[i] >> 8);
    }
  }
  __syncthreads();
  const int nt = min(N - tile * SORT_TILE, SORT_TILE);
  constexpr int PER = SORT_TILE / 256;
  // every source read is issued before the first store (clamped entries
  // past the tile's end are read and not stored)
  int tv[PER], dv[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = min(threadIdx.x + 256 * r, nt - 1);
    tv[r] = s_tok[i];
    dv[r] = s_dst[i];
  }
  if (src_map) {
#pragma unroll
    for (int r = 0; r < PER; ++r) tv[r] = src_map[(size_t)bh * N + tv[r]];
  }
#pragma unroll
  for (int r = 0; r < PER; ++r)
    if (threadIdx.x + 256 * r < nt) pb[dv[r]] = tv[r];
  if (slab_out) {
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (threadIdx.x + 256 * r < nt) slab_out[(size_t)bh * N + dv[r]] = s_lab[threadIdx.x + 256 * r];
  }
}

// --------------------------------------------------------------------------
// Fixed-point values for the exact k-means sums (rounds after the first
// three): v -> rint(v * 2^s), one power-of-two shift s per head.  With r2 a
// bound on max ||x||^2 < 2^E2, every |x_d| < 2^e with e = ceil(E2 / 2), so
// s = 30 - e keeps each value inside int32 and a sum of N < 2^24 of them
// inside int64; integer sums are exact, so they do not depend on the order
// of the additions.  The absolute error of a value is at most 2^(e - 31).
// --------------------------------------------------------------------------
__device__ __forceinline__ uint32_t km_r2_bits(const uint32_t* __restrict__ r2max, int bh) {
  uint32_t b = 0;
  for (int i = 0; i < KM_MSLOTS; ++i) b = max(b, r2max[bh * KM_MSLOTS + i]);
  return b;
}

__device__ __forceinline__ int km_fx_shift(uint32_t r2_bits) {
  const int E = (int)((r2_bits >> 23) & 0xff);
  const int E2 = (E ? E : 1) - 126;  // r2 < 2^E2
  return KM_FX_BITS - ((E2 + 1) >> 1);
}

__device__ __forceinline__ int km_fx_q(float v, int s) { return (int)rintf(ldexpf(v, s)); }

// --------------------------------------------------------------------------
// segment sums over the permuted order: chunk k of cluster c sums rows
// [offsets[c] + k' * rows, ...) of x[perm[.]] (k' = k - chunk_start[c]),
// optionally writing the permuted copy.  Fixed row-to-lane mapping and a
// fixed reduction order keep the sums deterministic.  SQ: sums of squared
// deviations from the cluster means `center` instead (variances).  PERM:
// the permuted copy x_perm is written (svgear_centroids); without it the
// kernel only reads (the k-means update).
// --------------------------------------------------------------------------
template <typename T, int D, bool SQ = false, bool FX = false, bool PERM = false>
__global__ void __launch_bounds__(256) km_partial_kernel(const T* __restrict__ x, const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ chunk_start, int N, int C,
                                                         int rows, int maxch, float* __restrict__ partial,
                                                         T* __restrict__ x_perm, const float* __restrict__ center = nullptr,
                                                         long long* __restrict__ pfx = nullptr,
                                                         const uint32_t* __restrict__ r2max = nullptr) {
  constexpr int EPL = 16 / sizeof(T);     // elements per lane (one 16-byte load)
  constexpr int LPR = D / EPL;            // lanes per row
  constexpr int RPI = 256 / LPR;          // rows per iteration
  using Acc = std::conditional_t<FX, long long, float>;
  __shared__ Acc red[RPI * D];
  __shared__ int s_c;
  const int bh = blockIdx.y, k = blockIdx.x;
  const int32_t* cs = chunk_start + (size_t)bh * (C + 1);
  if (k >= cs[C]) return;
  block_upper_index(cs, C, k, &s_c);
  __syncthreads();
  const int c = min(max(s_c, 0), C - 1);  // (in range even for a malformed table)
  const int32_t* off = offsets + (size_t)bh * (C + 1);
  const int r0 = off[c] + (k - cs[c]) * rows;
  const int r1 = min(r0 + rows, off[c + 1]);
  const int g = threadIdx.x / LPR, e0 = (threadIdx.x % LPR) * EPL;
  const T* xb = x + (size_t)bh * N * D;
  const int32_t* pb = perm + (size_t)bh * N;
  T* xpb = PERM ? x_perm + (size_t)bh * N * D : nullptr;
  Acc acc[EPL];
  float mu[EPL];
  const int fs = FX ? km_fx_shift(km_r2_bits(r2max, bh)) : 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    acc[e] = 0;
    mu[e] = SQ ? center[((size_t)bh * C + c) * D + e0 + e] : 0.f;
  }
  auto add = [&](float v, int e) {
    if constexpr (FX) {
      acc[e] += km_fx_q(v, fs);
    } else if constexpr (SQ) {
      const float dv = v - mu[e];
      acc[e] = fmaf(dv, dv, acc[e]);
    } else {
      acc[e] += v;
    }
  };
  int p = r0 + g;
  for (; p + 3 * RPI < r1; p += 4 * RPI) {
    int src[4];
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) src[k] = pb[p + k * RPI];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ld16(xb + (size_t)src[k] * D + e0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (PERM) st16(xpb + (size_t)(p + k * RPI) * D + e0, v[k]);
      const T* tv = reinterpret_cast<const T*>(&v[k]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) add(to_f32(tv[e]), e);
    }
  }
  if (p < r1) {
    // the last (fewer than 4) row steps, their loads in flight together:
    // steps past r1 read row r1 - 1 again and are dropped
    int src[4];
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) src[k] = pb[min(p + k * RPI, r1 - 1)];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ld16(xb + (size_t)src[k] * D + e0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // every value is added (a dropped step adds one that contributes
      // nothing), so no load can sink below the step's test
      const bool ok = p + k * RPI < r1;
      if constexpr (PERM)
        if (ok) st16(xpb + (size_t)(p + k * RPI) * D + e0, v[k]);
      const T* tv = reinterpret_cast<const T*>(&v[k]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) add(ok ? to_f32(tv[e]) : (SQ ? mu[e] : 0.f), e);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red[g * D + e0 + e] = acc[e];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 256) {
    Acc s = 0;
    for (int gg = 0; gg < RPI; ++gg) s += red[gg * D + d];
    if constexpr (FX) pfx[((size_t)bh * maxch + k) * D + d] = s;
    else partial[((size_t)bh * maxch + k) * D + d] = s;
  }
}

// means[c] = (sum of c's chunks, in order) / |c|.  Empty clusters: keep the
// old value (k-means update) or write 0 (svgear_centroids).  Each thread
// owns four consecutive columns of one cluster (D is a multiple of 4).
// With fx set (the last full round of a k-means call that continues with
// incremental rounds), the chunk sums are the fixed-point integers of
// km_partial_kernel<..., FX>: their total goes to fx, the cluster size to
// fxcnt, and the mean is taken from fx the way the incremental update takes
// it.
__global__ void __launch_bounds__(256) km_finalize_kernel(const float* __restrict__ partial,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ chunk_start, int C, int D,
                                                          int maxch, float* __restrict__ means, int keep_empty,
                                                          long long* __restrict__ fx = nullptr,
                                                          int32_t* __restrict__ fxcnt = nullptr,
                                                          const long long* __restrict__ pfx = nullptr,
                                                          const uint32_t* __restrict__ r2max = nullptr) {
  const int bh = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= C * D) return;
  const int c = i / D, d = i - c * D;
  const int32_t* off = offsets + (size_t)bh * (C + 1);
  const int32_t* cs = chunk_start + (size_t)bh * (C + 1);
  const int n = off[c + 1] - off[c];
  float* out = means + ((size_t)bh * C + c) * D + d;
  long long* fo = fx ? fx + ((size_t)bh * C + c) * D + d : nullptr;
  if (fx && d == 0) fxcnt[(size_t)bh * C + c] = n;
  if (n == 0) {
    if (!keep_empty)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = 0.f;
    if (fo)
#pragma unroll
      for (int e = 0; e < 4; ++e) fo[e] = 0;
    return;
  }
  // chunks added in order; eight loads are issued before their adds
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int k = cs[c];
  const int k1 = cs[c + 1];
  if (fo) {
    long long q[4] = {0, 0, 0, 0};
    const long long* pq = pfx + (size_t)bh * maxch * D + d;
    for (; k < k1; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] += pq[(size_t)k * D + e];
    const int fs = km_fx_shift(km_r2_bits(r2max, bh));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fo[e] = q[e];
      out[e] = (float)(ldexp((double)q[e], -fs) / (double)n);
    }
    return;
  }
  const float4* pp = reinterpret_cast<const float4*>(partial + (size_t)bh * maxch * D + d);
  const int stride = D / 4;
  auto add4 = [&](const float4& v) {
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  };
  for (; k + 8 <= k1; k += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = pp[(size_t)(k + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) add4(v[j]);
  }
  for (; k < k1; ++k) add4(pp[(size_t)k * stride]);
  const float fn = (float)n;
  out[0] = s.x / fn;
  out[1] = s.y / fn;
  out[2] = s.z / fn;
  out[3] = s.w / fn;
}

static void launch_finalize(const float* partial, const int32_t* offsets, const int32_t* cs, int BH, int C, int D,
                            int maxch, float* means, int keep_empty, hipStream_t st) {
  hipLaunchKernelGGL(km_finalize_kernel, dim3(cdiv(C * D / 4, 256), BH), dim3(256), 0, st, partial, offsets, cs, C,
                     D, maxch, means, keep_empty);
}

// --------------------------------------------------------------------------
// incremental update (rounds after the first three): only tokens whose label
// changed touch the sums.  Each workgroup owns kcl <= KD_CL clusters, picks
// from the moved list the entries that enter or leave them, adds the
// fixed-point values +-rint(x * 2^s) into LDS integer accumulators (exact, so
// the order of the list and of the atomics does not matter), then updates
// the owned clusters' fixed-point sums, sizes and means.  Clusters no entry
// touched keep everything.
// --------------------------------------------------------------------------
constexpr int KD_CL = 8;      // most clusters per workgroup
constexpr int KD_WIN = 1024;  // moved entries examined per window (4 per thread)

template <typename T, int D>
__global__ void __launch_bounds__(256) km_delta_kernel(const T* __restrict__ x, const int2* __restrict__ moved,
                                                       const int32_t* __restrict__ mtot,
                                                       const uint32_t* __restrict__ r2max, int N, int C, int kcl,
                                                       long long* __restrict__ fx, int32_t* __restrict__ fxcnt,
                                                       float* __restrict__ cent, uint32_t* __restrict__ nmax) {
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int RPI = 256 / LPR;       // rows per iteration
  constexpr int UR = 4;                // rows per thread loaded together
  __shared__ unsigned long long acc[KD_CL * D];
  __shared__ int s_m[2 * KD_WIN];  // token | local cluster << 24 | leaving << 27
  __shared__ int s_dc[KD_CL], s_cnt[KD_CL], s_nm;
  const int bh = blockIdx.y, c0 = blockIdx.x * kcl, tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) nmax[bh] = 0u;  // the assign kernel of this round has finished
  const int cap = km_mcap(N);
  const int2* mb = moved + (size_t)bh * KM_MSLOTS * cap;
  // the owned clusters' sums and sizes are loaded with the list lengths
  constexpr int FPT = KD_CL * D / 256;  // owned sum entries per thread
  long long fxv[FPT];
#pragma unroll
  for (int j = 0; j < FPT; ++j) {
    const int i = tid + 256 * j, c = c0 + i / D;
    fxv[j] = (i < kcl * D && c < C) ? fx[((size_t)bh * C + c0) * D + i] : 0;
  }
  const int cnt0 = (tid < kcl && c0 + tid < C) ? fxcnt[(size_t)bh * C + c0 + tid] : 0;
  // the list is the concatenation of the sub-lists: s_pre[i] = start of
  // sub-list i, s_pre[KM_MSLOTS] = length (one wave scans the counts)
  __shared__ int s_pre[KM_MSLOTS + 1];
  static_assert(KM_MSLOTS == SV_WAVE, "one sub-list count per lane of the first wave");
  if (tid < SV_WAVE) {
    const int v = mtot[bh * KM_MSLOTS + tid];
    int x = v;
#pragma unroll
    for (int o = 1; o < SV_WAVE; o <<= 1) {
      const int y = __shfl_up(x, o, SV_WAVE);
      if (tid >= o) x += y;
    }
    s_pre[tid] = x - v;
    if (tid == SV_WAVE - 1) s_pre[KM_MSLOTS] = x;
  }
  __syncthreads();
  const int M = s_pre[KM_MSLOTS];
  if (M == 0) return;
  auto entry = [&](int idx) {  // last sub-list starting at or before idx
    int lo = 0, hi = KM_MSLOTS - 1;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= idx) lo = mid; else hi = mid - 1;
    }
    return mb[(size_t)lo * cap + (idx - s_pre[lo])];
  };
  for (int i = tid; i < KD_CL * D; i += 256) acc[i] = 0ull;
  if (tid < KD_CL) s_dc[tid] = 0;
  const int fs = km_fx_shift(km_r2_bits(r2max, bh));
  const T* xb = x + (size_t)bh * N * D;
  const int g = tid / LPR, e0 = (tid % LPR) * EPL;
  int touched = 0;  // per-thread bit mask of owned clusters seen
  for (int w0 = 0; w0 < M; w0 += KD_WIN) {
    if (tid == 0) s_nm = 0;
    __syncthreads();
    int2 ev[KD_WIN / 256];
#pragma unroll
    for (int j = 0; j < KD_WIN / 256; ++j) {
      const int idx = w0 + tid + 256 * j;
      ev[j] = idx < M ? entry(idx) : make_int2(0, -1);
    }
#pragma unroll
    for (int j = 0; j < KD_WIN / 256; ++j) {
      if (ev[j].y < 0) continue;
      const int lo = (ev[j].y & 0xffff) - c0, ln = (ev[j].y >> 16) - c0;
      if ((unsigned)ln < (unsigned)kcl) s_m[atomicAdd(&s_nm, 1)] = ev[j].x | (ln << 24);
      if ((unsigned)lo < (unsigned)kcl) s_m[atomicAdd(&s_nm, 1)] = ev[j].x | (lo << 24) | (1 << 27);
    }
    __syncthreads();
    const int nm = s_nm;
    for (int r0 = 0; r0 < nm; r0 += UR * RPI) {
      int code[UR];
      u32x4 v[UR];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        // every load is issued (an empty slot reads row 0, unused), so the
        // UR rows are in flight together
        const int r = r0 + u * RPI + g;
        code[u] = r < nm ? s_m[r] : -1;
        v[u] = ld16(xb + (size_t)(code[u] >= 0 ? code[u] & 0xffffff : 0) * D + e0);
      }
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        if (code[u] < 0) continue;
        const int lc = (code[u] >> 24) & 7;
        const bool leave = (code[u] >> 27) & 1;
        const T* tv = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const long long q = km_fx_q(to_f32(tv[e]), fs);
          atomicAdd(&acc[lc * D + e0 + e], (unsigned long long)(leave ? -q : q));
        }
        if (e0 == 0) atomicAdd(&s_dc[lc], leave ? -1 : 1);
        touched |= 1 << lc;
      }
    }
    __syncthreads();
  }
  // which owned clusters any entry touched (each thread saw a subset)
  __shared__ int s_touch;
  if (tid == 0) s_touch = 0;
  __syncthreads();
  if (touched) atomicOr(&s_touch, touched);
  __syncthreads();
  const int tmask = s_touch;
  if (tid < kcl && ((tmask >> tid) & 1) && c0 + tid < C) {
    const int n = cnt0 + s_dc[tid];
    fxcnt[(size_t)bh * C + c0 + tid] = n;
    s_cnt[tid] = n;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < FPT; ++j) {
    const int i = tid + 256 * j;
    const int lc = i / D, c = c0 + lc;
    if (i >= kcl * D || c >= C || !((tmask >> lc) & 1)) continue;
    const size_t o = ((size_t)bh * C + c0) * D + i;
    const long long q = fxv[j] + (long long)acc[i];
    fx[o] = q;
    const int n = s_cnt[lc];
    if (n > 0) cent[o] = (float)(ldexp((double)q, -fs) / (double)n);  // an emptied cluster keeps its centroid
  }
}

// ---------------------------------------------------------------- host side
struct KmPlan {
  int BH, Cpad, ib, ntiles, maxch;
  size_t off_ops, off_nmax, off_counts, off_cs, off_partial, off_pfx, off_fx, off_fxcnt, off_moved, off_mtot, off_r2max;
  size_t off_cnorm, off_lb, off_slab, off_slab2, off_perm2, total;
  bool prune;  // candidate pruning in the tracking rounds (bf16 tokens only)
  int ibp;     // key index bits of the pruned assign (list positions < Cpad + 32)
};


static KmPlan km_plan(int B, int H, int N, int D, int C) {
  KmPlan p;
  p.BH = B * H;
  p.Cpad = round_up(C, 32);
  p.ib = bit_length((unsigned)(p.Cpad - 1));
  if (p.ib < 1) p.ib = 1;
  p.ntiles = cdiv(N, SORT_TILE);
  p.maxch = cdiv(N, MEAN_ROWS) + C;
  Carver cv(nullptr);
  p.off_ops = cv.used; cv.take<bf16>((size_t)p.BH * p.Cpad * (2 * D + KM_EXTRA));
  p.off_nmax = cv.used; cv.take<uint32_t>(p.BH);
  p.off_counts = cv.used; cv.take<int32_t>((size_t)p.BH * p.ntiles * C);
  p.off_cs = cv.used; cv.take<int32_t>((size_t)p.BH * (C + 1));
  p.off_partial = cv.used; cv.take<float>((size_t)p.BH * p.maxch * D);
  p.off_pfx = cv.used; cv.take<long long>((size_t)p.BH * p.maxch * D);
  p.off_fx = cv.used; cv.take<long long>((size_t)p.BH * C * D);
  p.off_fxcnt = cv.used; cv.take<int32_t>((size_t)p.BH * C);
  p.off_moved = cv.used; cv.take<int2>((size_t)p.BH * KM_MSLOTS * km_mcap(N));
  p.off_mtot = cv.used; cv.take<int32_t>((size_t)p.BH * KM_MSLOTS);
  p.off_r2max = cv.used; cv.take<uint32_t>((size_t)p.BH * KM_MSLOTS);
  p.prune = C >= KM_PRUNE_MIN_C && C <= KM_PRUNE_MAX_C;
  p.ibp = bit_length((unsigned)(p.Cpad + 31));
  p.off_cnorm = cv.used; if (p.prune) cv.take<float>((size_t)p.BH * p.Cpad);
  p.off_lb = cv.used; if (p.prune) cv.take<float>((size_t)p.BH * C * C);
  p.off_slab = cv.used; if (p.prune) cv.take<int32_t>((size_t)p.BH * N);
  p.off_slab2 = cv.used; if (p.prune) cv.take<int32_t>((size_t)p.BH * N);
  p.off_perm2 = cv.used; if (p.prune) cv.take<int32_t>((size_t)p.BH * N);
  p.total = cv.used;
  return p;
}

struct MeanPlan {
  int BH, maxch;
  size_t off_cs, off_partial, total;
};

static MeanPlan mean_plan(int B, int H, int N, int D, int C) {
  MeanPlan p;
  p.BH = B * H;
  p.maxch = cdiv(N, MEAN_ROWS) + C;
  Carver cv(nullptr);
  p.off_cs = cv.used; cv.take<int32_t>((size_t)p.BH * (C + 1));
  p.off_partial = cv.used; cv.take<float>((size_t)p.BH * p.maxch * D);
  p.total = cv.used;
  return p;
}

template <typename T, int D>
static void launch_partial(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* cs, int BH,
                           int N, int C, int maxch, float* partial, void* x_perm, hipStream_t st) {
  if (x_perm)
    hipLaunchKernelGGL((km_partial_kernel<T, D, false, false, true>), dim3(maxch, BH), dim3(256), 0, st, (const T*)x,
                       perm, offsets, cs, N, C, MEAN_ROWS, maxch, partial, (T*)x_perm, nullptr);
  else
    hipLaunchKernelGGL((km_partial_kernel<T, D>), dim3(maxch, BH), dim3(256), 0, st, (const T*)x, perm, offsets, cs,
                       N, C, MEAN_ROWS, maxch, partial, (T*)nullptr, nullptr);
}

template <typename T, int D>
static void launch_partial_sq(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* cs, int BH,
                              int N, int C, int maxch, float* partial, const float* means, hipStream_t st) {
  hipLaunchKernelGGL((km_partial_kernel<T, D, true>), dim3(maxch, BH), dim3(256), 0, st, (const T*)x, perm, offsets,
                     cs, N, C, MEAN_ROWS, maxch, partial, (T*)nullptr, means);
}

// The pruned assign exists for bf16 tokens only.
template <typename T, int D>
static void launch_assign_pruned(const void* x, const bf16* ops, const uint32_t* nmax, const float* cent, int N,
                                 int C, int Cpad, int ib, int32_t* labels, int2* moved, int32_t* mtot,
                                 const int32_t* perm, const float* lb, int32_t* slab, int BH, hipStream_t st) {
  // the candidate test takes CPT centroids per thread (C <= 256 CPT)
  if constexpr (sizeof(T) == 2) {
    if (C <= 512)
      hipLaunchKernelGGL((km_assign_kernel<T, D, true, 2>), dim3(cdiv(N, KM_TOK_WG), BH), dim3(256), 0, st,
                         (const T*)x, ops, nmax, cent, N, C, Cpad, ib, labels, moved, mtot, nullptr, perm, lb, slab,
                         slab);
    else
      hipLaunchKernelGGL((km_assign_kernel<T, D, true, KM_PRUNE_MAX_C / 256>), dim3(cdiv(N, KM_TOK_WG), BH),
                         dim3(256), 0, st, (const T*)x, ops, nmax, cent, N, C, Cpad, ib, labels, moved, mtot, nullptr,
                         perm, lb, slab, slab);
  }
}

// labels[order[p]] = lab_by_pos[p]: token-order labels from an order grouped by label
__global__ void __launch_bounds__(256) km_unsort_kernel(const int32_t* __restrict__ order,
                                                        const int32_t* __restrict__ lab_by_pos, int N,
                                                        int32_t* __restrict__ labels) {
  const int bh = blockIdx.y, q = blockIdx.x * 256 + threadIdx.x;
  if (q < N) labels[(size_t)bh * N + order[(size_t)bh * N + q]] = lab_by_pos[(size_t)bh * N + q];
}

template <typename T, int D>
static svgear_status kmeans_impl(const void* x, int BH, int N, int C, int iters, float* cent, int32_t* labels,
                                 int32_t* perm, int32_t* offsets, char* ws, const KmPlan& p, hipStream_t st) {
  bf16* ops = reinterpret_cast<bf16*>(ws + p.off_ops);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
  int32_t* cs = reinterpret_cast<int32_t*>(ws + p.off_cs);
  float* partial = reinterpret_cast<float*>(ws + p.off_partial);
  uint32_t* nmax = reinterpret_cast<uint32_t*>(ws + p.off_nmax);
  long long* pfx = reinterpret_cast<long long*>(ws + p.off_pfx);
  long long* fx = reinterpret_cast<long long*>(ws + p.off_fx);
  int32_t* fxcnt = reinterpret_cast<int32_t*>(ws + p.off_fxcnt);
  int2* moved = reinterpret_cast<int2*>(ws + p.off_moved);
  int32_t* mtot = reinterpret_cast<int32_t*>(ws + p.off_mtot);
  uint32_t* r2max = reinterpret_cast<uint32_t*>(ws + p.off_r2max);
  float* cnorm = reinterpret_cast<float*>(ws + p.off_cnorm);
  float* lb = reinterpret_cast<float*>(ws + p.off_lb);
  // pruned rounds keep the tokens in an order grouped by label: pc[q] is the
  // token at position q and sc[q] its label; each round updates sc in place
  // and the next regroups (pc, sc) by it into the other pair of buffers
  int32_t* pc = perm;
  int32_t* sc = reinterpret_cast<int32_t*>(ws + p.off_slab);
  int32_t* pn = reinterpret_cast<int32_t*>(ws + p.off_perm2);
  int32_t* sn = reinterpret_cast<int32_t*>(ws + p.off_slab2);
  bool grouped = false;
  // candidate pruning of the tracking rounds (bf16 tokens, a few hundred centroids or more)
  const bool prune = p.prune && sizeof(T) == 2;
  // The first KM_FULL_ROUNDS updates recompute every sum from the sorted
  // tokens (the first rounds move many tokens); the last of them leaves
  // exact fixed-point sums, and every later round updates those from the
  // tokens whose label changed.
  const int nfull = iters > KM_FULL_ROUNDS ? KM_FULL_ROUNDS : iters;
  const bool incr = iters > nfull;
  // clusters per delta workgroup: enough workgroups to fill the chip
  const int kcl = std::max(1, std::min(KD_CL, cdiv(C * BH, 2048)));
  hipLaunchKernelGGL(km_clear_kernel, dim3(cdiv(BH, 256)), dim3(256), 0, st, nmax, BH);
  if (incr)
    hipLaunchKernelGGL(km_clear_kernel, dim3(cdiv(BH * KM_MSLOTS, 256)), dim3(256), 0, st, r2max, BH * KM_MSLOTS);
  (void)hipFuncSetAttribute((const void*)km_scatter_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)km_scatter_lds(C));
  auto sort_labels = [&]() {  // tile histograms -> offsets -> stable perm
    hipLaunchKernelGGL(km_hist_kernel, dim3(p.ntiles, BH), dim3(256), 0, st, labels, N, C, p.ntiles, counts);
    hipLaunchKernelGGL(km_scan_kernel, dim3(BH), dim3(1024), 0, st, counts, N, C, p.ntiles, MEAN_ROWS, offsets, cs,
                       nmax);
    hipLaunchKernelGGL(km_scatter_kernel, dim3(p.ntiles, BH), dim3(256), km_scatter_lds(C), st, labels, counts, N,
                       C, p.ntiles, p.ib, perm, nullptr, nullptr);
  };
  for (int it = 0; it < iters; ++it) {
    const bool track = it >= nfull;             // incremental round
    const bool setup = incr && it == nfull - 1;  // full round that sets up the fixed-point sums
    const bool pr = prune && track;
    if (pr) {
      // the tokens grouped by their current labels, with those labels by position
      const int32_t* src = grouped ? sc : labels;
      hipLaunchKernelGGL(km_hist_kernel, dim3(p.ntiles, BH), dim3(256), 0, st, src, N, C, p.ntiles, counts);
      hipLaunchKernelGGL(km_scan_kernel, dim3(BH), dim3(1024), 0, st, counts, N, C, p.ntiles, MEAN_ROWS, offsets,
                         cs, nmax);
      hipLaunchKernelGGL(km_scatter_kernel, dim3(p.ntiles, BH), dim3(256), km_scatter_lds(C), st, src, counts, N,
                         C, p.ntiles, p.ib, grouped ? pn : pc, grouped ? pc : nullptr, grouped ? sn : sc);
      if (grouped) {
        std::swap(pc, pn);
        std::swap(sc, sn);
      }
      grouped = true;
    }
    hipLaunchKernelGGL((km_prep_kernel<D>), dim3(cdiv(p.Cpad, KM_PREP_ROWS), BH), dim3(256), 0, st, cent, C, p.Cpad,
                       ops, nmax, track ? mtot : nullptr, pr ? cnorm : nullptr);
    if (pr) {
      const int nt = p.Cpad / 32;
      hipLaunchKernelGGL((km_cc_kernel<D>), dim3(cdiv(nt * nt, 4), BH), dim3(256), 0, st, ops, cnorm, C, p.Cpad, lb);
      launch_assign_pruned<T, D>(x, ops, nmax, cent, N, C, p.Cpad, p.ibp, labels, moved, mtot, pc, lb, sc, BH, st);
    } else {
      hipLaunchKernelGGL((km_assign_kernel<T, D>), dim3(cdiv(N, KM_TOK_WG), BH), dim3(256), 0, st, (const T*)x, ops,
                         nmax, cent, N, C, p.Cpad, p.ib, labels, track ? moved : nullptr, mtot,
                         setup ? r2max : nullptr, nullptr, nullptr, nullptr, nullptr);
    }
    if (track) {
      hipLaunchKernelGGL((km_delta_kernel<T, D>), dim3(cdiv(C, kcl), BH), dim3(256), 0, st, (const T*)x, moved, mtot,
                         r2max, N, C, kcl, fx, fxcnt, cent, nmax);
    } else if (setup) {
      sort_labels();
      hipLaunchKernelGGL((km_partial_kernel<T, D, false, true>), dim3(p.maxch, BH), dim3(256), 0, st, (const T*)x,
                         perm, offsets, cs, N, C, MEAN_ROWS, p.maxch, partial, (T*)nullptr, nullptr, pfx, r2max);
      hipLaunchKernelGGL(km_finalize_kernel, dim3(cdiv(C * D / 4, 256), BH), dim3(256), 0, st, partial, offsets, cs,
                         C, D, p.maxch, cent, 1, fx, fxcnt, pfx, r2max);
    } else {
      sort_labels();
      launch_partial<T, D>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, nullptr, st);
      launch_finalize(partial, offsets, cs, BH, C, D, p.maxch, cent, 1, st);
    }
  }
  if (grouped)  // the last labels back in token order
    hipLaunchKernelGGL(km_unsort_kernel, dim3(cdiv(N, 256), BH), dim3(256), 0, st, pc, sc, N, labels);
  if (incr) sort_labels();  // perm and offsets of the last labels
  return check_launch("svgear_kmeans");
}

}  // namespace svg

using namespace svg;

extern "C" size_t svgear_kmeans_workspace(int B, int H, int N, int D, int C) {
  if (B < 1 || H < 1 || N < 1 || C < 1 || (D != 64 && D != 128)) return 0;
  return km_plan(B, H, N, D, C).total;
}

extern "C" svgear_status svgear_kmeans(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C, int iters,
                                       float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  svgear_status st = check_common("kmeans", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (C < 1 || C > N || C > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "kmeans: C=%d must be in [1, min(N=%d, %d)]", C, N, SVGEAR_MAX_CLUSTERS);
  if (iters < 1) return fail(SVGEAR_ERR_INVALID_ARG, "kmeans: iters=%d must be >= 1", iters);
  if (!x || !centroids || !labels || !perm || !offsets) return fail(SVGEAR_ERR_INVALID_ARG, "kmeans: null pointer");
  KmPlan p = km_plan(B, H, N, D, C);
  st = check_ws("kmeans", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  const int BH = B * H;
  if (dt == SVGEAR_BF16)
    return D == 128 ? kmeans_impl<bf16, 128>(x, BH, N, C, iters, centroids, labels, perm, offsets, w, p, stream)
                    : kmeans_impl<bf16, 64>(x, BH, N, C, iters, centroids, labels, perm, offsets, w, p, stream);
  return D == 128 ? kmeans_impl<float, 128>(x, BH, N, C, iters, centroids, labels, perm, offsets, w, p, stream)
                  : kmeans_impl<float, 64>(x, BH, N, C, iters, centroids, labels, perm, offsets, w, p, stream);
}

extern "C" size_t svgear_centroids_workspace(int B, int H, int N, int D, int C) {
  if (B < 1 || H < 1 || N < 1 || C < 1 || (D != 64 && D != 128)) return 0;
  return mean_plan(B, H, N, D, C).total;
}

extern "C" svgear_status svgear_centroids(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                                          const int32_t* perm, const int32_t* offsets, void* x_perm, float* means,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  svgear_status st = check_common("centroids", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (C < 1 || C > N || C > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "centroids: C=%d must be in [1, min(N=%d, %d)]", C, N, SVGEAR_MAX_CLUSTERS);
  if (!x || !perm || !offsets) return fail(SVGEAR_ERR_INVALID_ARG, "centroids: null pointer");
  if (!x_perm && !means) return SVGEAR_OK;
  MeanPlan p = mean_plan(B, H, N, D, C);
  st = check_ws("centroids", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  int32_t* cs = reinterpret_cast<int32_t*>(w + p.off_cs);
  float* partial = reinterpret_cast<float*>(w + p.off_partial);
  const int BH = B * H;
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, offsets, C, MEAN_ROWS, cs);
  if (dt == SVGEAR_BF16) {
    if (D == 128) launch_partial<bf16, 128>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, x_perm, stream);
    else launch_partial<bf16, 64>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, x_perm, stream);
  } else {
    if (D == 128) launch_partial<float, 128>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, x_perm, stream);
    else launch_partial<float, 64>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, x_perm, stream);
  }
  if (means)
    launch_finalize(partial, offsets, cs, BH, C, D, p.maxch, means, 0, stream);
  return check_launch("svgear_centroids");
}

extern "C" svgear_status svgear_centroid_variances(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                                                   const int32_t* perm, const int32_t* offsets, const float* means,
                                                   float* vars, void* ws, size_t ws_bytes, hipStream_t stream) {
  svgear_status st = check_common("centroid_variances", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (C < 1 || C > N || C > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "centroid_variances: C=%d must be in [1, min(N=%d, %d)]", C, N,
                SVGEAR_MAX_CLUSTERS);
  if (!x || !perm || !offsets || !means || !vars) return fail(SVGEAR_ERR_INVALID_ARG, "centroid_variances: null pointer");
  MeanPlan p = mean_plan(B, H, N, D, C);
  st = check_ws("centroid_variances", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  int32_t* cs = reinterpret_cast<int32_t*>(w + p.off_cs);
  float* partial = reinterpret_cast<float*>(w + p.off_partial);
  const int BH = B * H;
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, offsets, C, MEAN_ROWS, cs);
  if (dt == SVGEAR_BF16) {
    if (D == 128) launch_partial_sq<bf16, 128>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, means, stream);
    else launch_partial_sq<bf16, 64>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, means, stream);
  } else {
    if (D == 128) launch_partial_sq<float, 128>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, means, stream);
    else launch_partial_sq<float, 64>(x, perm, offsets, cs, BH, N, C, p.maxch, partial, means, stream);
  }
  launch_finalize(partial, offsets, cs, BH, C, D, p.maxch, vars, 0, stream);
  return check_launch("svgear_centroid_variances");
}
