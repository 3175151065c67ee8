// Error-aware routing: svgear_route.
//
// FrontierCS blog on SVG-EAR, probe paragraph: the query cluster's mean
// q_bar_i scores every real key k of block (i, j), s_ik = q_bar_i.k * scale,
// and the block's error is e_ij = sum_{k in K_j} || e^{s_bar_ij} v_bar_j -
// e^{s_ik} v_k ||^2 (taken relative to the row maximum M_i = max_k s_ik);
// dividing by the block's token pairs gives the ratio the greedy fill ranks
// (Pith review, "What carries the argument").
//
// Evaluation.  With ds_k = s_ik - s_bar_ij = scale * q_bar_i.(k - k_bar_j), a
// piece-local stabiliser delta >= max(0, max_k ds_k), a = e^{-delta},
// b_k = e^{ds_k - delta} and eps_k = b_k - a, each key's term expands exactly as
//   || a v_bar - b_k v_k ||^2 = a^2 ||v_bar - v_k||^2 - 2 a eps_k w_k + eps_k^2 ||v_k||^2,
//   w_k = (v_bar - v_k).v_k,
// so per (query cluster, key) only three scalars are accumulated: the error
// term is never formed in d dimensions per query, and ds_k comes from an MFMA
// of the centred keys (k - k_bar_j, split hi/lo in bf16) against q_bar (hi/lo),
// which keeps the exponent accurate where e^{ds} is close to 1.  Pieces of a
// key cluster merge by rescaling to the larger stabiliser; the row maximum is
// M_i = max_j (s_bar_ij + delta_ij), and e_ij = e^{2 (s_bar_ij + delta_ij - M_i)}
// (a^2 T1 - 2 a S2 + S3).
#include "common.h"
#include "host.h"
#include "scan.h"

namespace svg {

constexpr int RT_PIECE = 512;  // keys per workgroup piece
constexpr int RT_QB = 128;     // query clusters per LDS block
constexpr int SEL_MAX = SVGEAR_MAX_CLUSTERS;

// q_bar split in bf16 hi/lo, padded to a multiple of 32 rows with zeros.
template <int D>
__global__ void __launch_bounds__(256) rt_prep_kernel(const float* __restrict__ qm, int Cq, int Cqp,
                                                      bf16* __restrict__ qhi, bf16* __restrict__ qlo) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= Cqp * D) return;
  const int row = i / D;
  const float v = row < Cq ? qm[(size_t)bh * Cq * D + i] : 0.f;
  bf16 h, l;
  split_bf16(v, h, l);
  qhi[(size_t)bh * Cqp * D + i] = h;
  qlo[(size_t)bh * Cqp * D + i] = l;
}

// s_bar[i][j] = scale * q_bar_i . k_bar_j in fp64, rounded to fp32.  A block
// computes a 16 x 64 tile from rows staged in LDS (row stride D + 1 floats).
__global__ void __launch_bounds__(256) rt_sbar_kernel(const float* __restrict__ qm, const float* __restrict__ km,
                                                      int Cq, int Ck, int D, float scale, float* __restrict__ sbar) {
  __shared__ float sq[16 * 129];
  __shared__ float sk[64 * 129];
  const int bh = blockIdx.z, i0 = blockIdx.y * 16, j0 = blockIdx.x * 64, tid = threadIdx.x;
  const int S = D + 1;
  for (int v = tid; v < 16 * D; v += 256) {
    const int r = v / D, d = v - r * D;
    sq[r * S + d] = (i0 + r < Cq) ? qm[((size_t)bh * Cq + i0 + r) * D + d] : 0.f;
  }
  for (int v = tid; v < 64 * D; v += 256) {
    const int r = v / D, d = v - r * D;
    sk[r * S + d] = (j0 + r < Ck) ? km[((size_t)bh * Ck + j0 + r) * D + d] : 0.f;
  }
  __syncthreads();
  const int jj = tid & 63, ig = tid >> 6;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int d = 0; d < D; ++d) {
    const double kv = (double)sk[jj * S + d];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += (double)sq[(ig * 4 + r) * S + d] * kv;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + ig * 4 + r, j = j0 + jj;
    if (i < Cq && j < Ck) sbar[((size_t)bh * Cq + i) * Ck + j] = (float)(acc[r] * (double)scale);
  }
}

// One workgroup per piece (<= RT_PIECE keys of one key cluster).  Output per
// (piece, query cluster): (delta, S2, S3); per piece: T1 = sum ||v_bar - v_k||^2.
template <typename T, int D>
__global__ void __launch_bounds__(256) rt_main_kernel(const T* __restrict__ kp, const T* __restrict__ vp,
                                                      const float* __restrict__ kmeans, const float* __restrict__ vmeans,
                                                      const int32_t* __restrict__ koff, const int32_t* __restrict__ pstart,
                                                      const bf16* __restrict__ qhi, const bf16* __restrict__ qlo,
                                                      int N, int Cq, int Cqp, int Ck, int maxp, float scale,
                                                      float* __restrict__ part, float* __restrict__ t1part) {
  constexpr int KS = D / 16;
  constexpr int SQ = D + 8;  // LDS row stride for q_bar (bf16)
  __shared__ __attribute__((aligned(1024))) bf16 s_qh[RT_QB * SQ];
  __shared__ __attribute__((aligned(1024))) bf16 s_ql[RT_QB * SQ];
  __shared__ float s_kbar[D], s_vbar[D];
  __shared__ __attribute__((aligned(16))) float s_w[4][32];
  __shared__ __attribute__((aligned(16))) float s_vv[4][32];
  __shared__ float s_st[4][RT_QB][3];
  __shared__ float s_t1[4];
  __shared__ int s_j;

  const int bh = blockIdx.y, pc = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int half = lane >> 5, col = lane & 31;
  const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
  if (pc >= ps[Ck]) return;
  if (tid == 0) s_j = upper_index(ps, Ck, pc);
  __syncthreads();
  const int j = s_j;
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int r0 = ko[j] + (pc - ps[j]) * RT_PIECE;
  const int r1 = min(r0 + RT_PIECE, ko[j + 1]);
  const int ntile = (r1 - r0 + 31) / 32;
  for (int d = tid; d < D; d += 256) {
    s_kbar[d] = kmeans[((size_t)bh * Ck + j) * D + d];
    s_vbar[d] = vmeans[((size_t)bh * Ck + j) * D + d];
  }
  const T* kb = kp + (size_t)bh * N * D;
  const T* vb = vp + (size_t)bh * N * D;
  float t1acc = 0.f;

  for (int qb = 0; qb < Cqp; qb += RT_QB) {
    const int nq = min(RT_QB, Cqp - qb);
    const int nqt = nq / 32;
    __syncthreads();
    {
      // q_bar hi/lo rows straight into LDS (no registers, one memory latency):
      // load j fills bytes [1024 j, 1024 j + 1024) of the padded block, lane
      // L the 16 bytes at o = 1024 j + 16 L, i.e. byte o % (2 SQ) of row
      // o / (2 SQ); pad bytes and rows past nq take row 0's first bytes
      constexpr int NJ = RT_QB * SQ * 2 / 1024;
      static_assert(RT_QB * SQ * 2 % 1024 == 0, "q_bar block must be whole 1 KB loads");
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(qhi + (size_t)bh * Cqp * D), (short)0, Cqp * D * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(qlo + (size_t)bh * Cqp * D), (short)0, Cqp * D * 2, 0x00020000);
      for (int j = w; j < NJ; j += 4) {
        const int o = 1024 * j + 16 * lane;
        const int r = o / (2 * SQ), cb = o - r * (2 * SQ);
        const int off = (r < nq && cb < 2 * D) ? (qb + r) * D * 2 + cb : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rh, (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(s_qh) + 1024 * j), 16, off, 0, 0,
            0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rl, (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(s_ql) + 1024 * j), 16, off, 0, 0,
            0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vector-memory count 0 (this wave's loads landed)
    }
    __syncthreads();
    float dl[4], s2[4], s3[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) { dl[qt] = 0.f; s2[qt] = 0.f; s3[qt] = 0.f; }

    for (int tl = w; tl < ntile; tl += 4) {
      const int p = r0 + tl * 32 + col;
      const bool ok = p < r1;
      bf16x8 ah[KS], al[KS];
      float wp = 0.f, vvp = 0.f, t1p = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = 16 * ks + 8 * half;
        float kf[8], vf[8];
        if constexpr (sizeof(T) == 2) {
          bf16x8 kv = {}, vv = {};
          if (ok) {
            kv = *reinterpret_cast<const bf16x8*>(kb + (size_t)p * D + d0);
            vv = *reinterpret_cast<const bf16x8*>(vb + (size_t)p * D + d0);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) { kf[e] = (float)kv[e]; vf[e] = (float)vv[e]; }
        } else {
          f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
          if (ok) {
            k0 = *reinterpret_cast<const f32x4*>(kb + (size_t)p * D + d0);
            k1 = *reinterpret_cast<const f32x4*>(kb + (size_t)p * D + d0 + 4);
            v0 = *reinterpret_cast<const f32x4*>(vb + (size_t)p * D + d0);
            v1 = *reinterpret_cast<const f32x4*>(vb + (size_t)p * D + d0 + 4);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) { kf[e] = k0[e]; kf[e + 4] = k1[e]; vf[e] = v0[e]; vf[e + 4] = v1[e]; }
        }
        bf16x8 h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dk = ok ? kf[e] - s_kbar[d0 + e] : 0.f;
          bf16 hh, ll;
          split_bf16(dk, hh, ll);
          h[e] = hh;
          l[e] = ll;
          const float dv = s_vbar[d0 + e] - vf[e];
          wp += dv * vf[e];
          vvp += vf[e] * vf[e];
          t1p += dv * dv;
        }
        ah[ks] = h;
        al[ks] = l;
      }
      wp += shfl_xor(wp, 32);
      vvp += shfl_xor(vvp, 32);
      t1p += shfl_xor(t1p, 32);
      if (!ok) { wp = 0.f; vvp = 0.f; t1p = 0.f; }
      if (qb == 0 && half == 0) t1acc += t1p;
      if (half == 0) { s_w[w][col] = wp; s_vv[w][col] = vvp; }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      float wv[16], vvv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&s_w[w][8 * g + 4 * half]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&s_vv[w][8 * g + 4 * half]);
#pragma unroll
        for (int e = 0; e < 4; ++e) { wv[4 * g + e] = a[e]; vvv[4 * g + e] = b[e]; }
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        if (qt < nqt) {
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int qrow = qt * 32 + col;
            const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(&s_qh[qrow * SQ + 16 * ks + 8 * half]);
            const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(&s_ql[qrow * SQ + 16 * ks + 8 * half]);
            acc = mfma_bf16(ah[ks], bh_, acc);
            acc = mfma_bf16(ah[ks], bl_, acc);
            acc = mfma_bf16(al[ks], bh_, acc);
          }
          float mx = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r] * scale);
          const float dn = fmaxf(dl[qt], mx);
          if (dn > dl[qt]) {
            const float f = __expf(dl[qt] - dn);
            s2[qt] *= f;
            s3[qt] *= f * f;
            dl[qt] = dn;
          }
          const float a = __expf(-dn);
          float t2 = 0.f, t3 = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float eps = __expf(acc[r] * scale - dn) - a;
            t2 = fmaf(eps, wv[r], t2);
            t3 = fmaf(eps * eps, vvv[r], t3);
          }
          s2[qt] += t2;
          s3[qt] += t3;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // merge the two halves (same queries, different keys), then the waves
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const float od = shfl_xor(dl[qt], 32), o2 = shfl_xor(s2[qt], 32), o3 = shfl_xor(s3[qt], 32);
      const float dm = fmaxf(dl[qt], od);
      const float fa = __expf(dl[qt] - dm), fb = __expf(od - dm);
      const float m2 = s2[qt] * fa + o2 * fb;
      const float m3 = s3[qt] * fa * fa + o3 * fb * fb;
      if (half == 0 && qt < nqt) {
        s_st[w][qt * 32 + col][0] = dm;
        s_st[w][qt * 32 + col][1] = m2;
        s_st[w][qt * 32 + col][2] = m3;
      }
    }
    __syncthreads();
    if (tid < nq && qb + tid < Cq) {
      float dm = s_st[0][tid][0];
      for (int ww = 1; ww < 4; ++ww) dm = fmaxf(dm, s_st[ww][tid][0]);
      float m2 = 0.f, m3 = 0.f;
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __expf(s_st[ww][tid][0] - dm);
        m2 += s_st[ww][tid][1] * f;
        m3 += s_st[ww][tid][2] * f * f;
      }
      float* o = part + (((size_t)bh * maxp + pc) * Cq + qb + tid) * 3;
      o[0] = dm;
      o[1] = m2;
      o[2] = m3;
    }
  }
  t1acc = wave_sum_f(t1acc);
  if (lane == 0) s_t1[w] = t1acc;
  __syncthreads();
  if (tid == 0) t1part[(size_t)bh * maxp + pc] = ((s_t1[0] + s_t1[1]) + s_t1[2]) + s_t1[3];
}

// One workgroup per (batch, head, query cluster): ratios r_ij, then the
// greedy fill.  Keys sort as (r descending, j ascending) by a bitonic sort of
// (~bits(r) << 32 | j); empty key clusters sort last and are never taken.
// Sort key of a non-negative score: larger scores first, ties to the lower
// index; NaN sorts first so that it cannot hide.
__device__ __forceinline__ uint64_t desc_key(float r, int j) {
  const uint32_t hi = (r != r) ? 0xFFFFFFFFu : ~__float_as_uint(r == 0.f ? 0.f : r);
  return ((uint64_t)hi << 32) | (uint32_t)j;
}

// Ascending bitonic sort of P (a power of two) keys in LDS by a 256-thread block.
__device__ __forceinline__ void block_sort_keys(uint64_t* s_key, int P) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= P; k <<= 1) {
    for (int s = k >> 1; s > 0; s >>= 1) {
      for (int t = tid; t < P; t += 256) {
        const int o = t ^ s;
        if (o > t) {
          const uint64_t a = s_key[t], b = s_key[o];
          const bool up = (t & k) == 0;
          if ((a > b) == up) { s_key[t] = b; s_key[o] = a; }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// SVG2 top-p over the centroid shares of one query cluster (SVG2 summary,
// "Centroid-Based Top-p Selection").  P'_j = n_j e^{S_j - M} / sum_l n_l e^{S_l - M}
// in fp64, M the largest S_j over non-empty clusters, rounded to fp32 (or taken
// from probs_in).  Non-empty clusters are ordered by (P' desc, j asc); one wave
// adds the shares in that order in fp64, one term at a time, and a cluster is
// taken while the sum before it is < p (p >= 1 takes them all).  Writes the
// mask row (nullable), the row's key budget = keys taken (nullable) and P'
// (nullable).
__global__ void __launch_bounds__(256) rt_topp_kernel(const float* __restrict__ sbar, const float* __restrict__ probs_in,
                                                      const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
                                                      int Cq, int Ck, double p, float* __restrict__ probs_out,
                                                      int32_t* __restrict__ budget, uint8_t* __restrict__ mask) {
  __shared__ uint64_t s_key[SEL_MAX];
  __shared__ float s_p[SEL_MAX];
  __shared__ int s_n[SEL_MAX];
  __shared__ double s_sum[4];
  __shared__ float s_max[4];
  __shared__ int s_take[2];
  const int bh = blockIdx.y, i = blockIdx.x, tid = threadIdx.x;
  const int32_t* qo = qoff + (size_t)bh * (Cq + 1);
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const size_t row = (size_t)bh * Cq + i;
  if (qo[i + 1] == qo[i]) {
    for (int j = tid; j < Ck; j += 256) {
      if (mask) mask[row * Ck + j] = 0;
      if (probs_out) probs_out[row * Ck + j] = 0.f;
    }
    if (tid == 0 && budget) budget[row] = 0;
    return;
  }
  for (int j = tid; j < Ck; j += 256) s_n[j] = ko[j + 1] - ko[j];
  if (probs_in) {
    for (int j = tid; j < Ck; j += 256) s_p[j] = probs_in[row * Ck + j];
  } else {
    const float* srow = sbar + row * Ck;
    float m = -INFINITY;
    for (int j = tid; j < Ck; j += 256)
      if (ko[j + 1] > ko[j]) m = fmaxf(m, srow[j]);
    m = wave_max_f(m);
    if (lane_id() == 0) s_max[wave_id()] = m;
    __syncthreads();
    const double M = (double)fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    double sum = 0.0;
    for (int j = tid; j < Ck; j += 256) {
      const int n = s_n[j];
      if (n > 0) sum += (double)n * exp((double)srow[j] - M);
    }
    sum = wave_sum_d(sum);
    if (lane_id() == 0) s_sum[wave_id()] = sum;
    __syncthreads();
    const double tot = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
    for (int j = tid; j < Ck; j += 256) {
      const int n = s_n[j];
      s_p[j] = n > 0 ? (float)((double)n * exp((double)srow[j] - M) / tot) : 0.f;
    }
  }
  __syncthreads();
  if (probs_out)
    for (int j = tid; j < Ck; j += 256) probs_out[row * Ck + j] = s_p[j];
  int P = 1;
  while (P < Ck) P <<= 1;
  for (int j = tid; j < P; j += 256) s_key[j] = (j < Ck && s_n[j] > 0) ? desc_key(s_p[j], j) : ~0ull;
  __syncthreads();
  block_sort_keys(s_key, P);
  if (tid < SV_WAVE) {
    double cum = 0.0;
    int taken = 0, keys = 0;
    bool stop = false;
    for (int t0 = 0; t0 < P && !stop; t0 += SV_WAVE) {
      const int t = t0 + tid;
      const uint64_t key = t < P ? s_key[t] : ~0ull;
      const bool valid = key != ~0ull;
      const int j = (int)(uint32_t)key;
      const double pv = valid ? (double)s_p[j] : 0.0;
      const int nv = valid ? s_n[j] : 0;
      const uint64_t vb = ballot(valid);
      for (int l = 0; l < SV_WAVE; ++l) {
        if (!((vb >> l) & 1ull) || (p < 1.0 && cum >= p)) { stop = true; break; }
        cum += readlane_d(pv, l);
        keys += __builtin_amdgcn_readlane(nv, l);
        ++taken;
      }
    }
    if (tid == 0) { s_take[0] = taken; s_take[1] = keys; }
  }
  __syncthreads();
  const int T = s_take[0];
  if (mask) {
    uint8_t* mrow = mask + row * Ck;
    for (int t = tid; t < P; t += 256) {
      const uint64_t key = s_key[t];
      if (key != ~0ull) mrow[(int)(uint32_t)key] = t < T ? 1 : 0;
    }
    for (int j = tid; j < Ck; j += 256)
      if (s_n[j] == 0) mrow[j] = 0;
  }
  if (tid == 0 && budget) budget[row] = s_take[1];
}

__global__ void __launch_bounds__(256) rt_select_kernel(const float* __restrict__ part, const float* __restrict__ t1part,
                                                        const int32_t* __restrict__ pstart, const float* __restrict__ sbar,
                                                        const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
                                                        const float* __restrict__ scores_in, int Cq, int Ck, int maxp,
                                                        double budget, const int32_t* __restrict__ row_budget,
                                                        float* __restrict__ scores_out, uint8_t* __restrict__ mask) {
  __shared__ uint64_t s_key[SEL_MAX];
  __shared__ float s_mu[SEL_MAX];
  __shared__ float s_e[SEL_MAX];
  __shared__ float s_red[4];
  __shared__ int s_scan[16];
  const int bh = blockIdx.y, i = blockIdx.x, tid = threadIdx.x;
  const int32_t* qo = qoff + (size_t)bh * (Cq + 1);
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int mi = qo[i + 1] - qo[i];
  uint8_t* mrow = mask + ((size_t)bh * Cq + i) * Ck;
  float* srow = scores_out ? scores_out + ((size_t)bh * Cq + i) * Ck : nullptr;
  if (mi == 0) {
    for (int j = tid; j < Ck; j += 256) {
      mrow[j] = 0;
      if (srow) srow[j] = 0.f;
    }
    return;
  }
  int P = 1;
  while (P < Ck) P <<= 1;
  if (scores_in) {
    const float* in = scores_in + ((size_t)bh * Cq + i) * Ck;
    for (int j = tid; j < Ck; j += 256) s_e[j] = in[j];
  } else {
    const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
    float mloc = -INFINITY;
    for (int j = tid; j < Ck; j += 256) {
      float mu = -INFINITY, E = 0.f;
      if (ko[j + 1] > ko[j]) {
        float dm = 0.f;
        for (int pc = ps[j]; pc < ps[j + 1]; ++pc) dm = fmaxf(dm, part[(((size_t)bh * maxp + pc) * Cq + i) * 3]);
        float S2 = 0.f, S3 = 0.f, T1 = 0.f;
        for (int pc = ps[j]; pc < ps[j + 1]; ++pc) {
          const float* o = part + (((size_t)bh * maxp + pc) * Cq + i) * 3;
          const float f = __expf(o[0] - dm);
          S2 += o[1] * f;
          S3 += o[2] * f * f;
          T1 += t1part[(size_t)bh * maxp + pc];
        }
        const float a = __expf(-dm);
        E = fmaxf(0.f, a * a * T1 - 2.f * a * S2 + S3);
        mu = sbar[((size_t)bh * Cq + i) * Ck + j] + dm;
        mloc = fmaxf(mloc, mu);
      }
      s_mu[j] = mu;
      s_e[j] = E;
    }
    mloc = wave_max_f(mloc);
    if (lane_id() == 0) s_red[wave_id()] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    for (int j = tid; j < Ck; j += 256) {
      const int nj = ko[j + 1] - ko[j];
      float r = 0.f;
      if (nj > 0) {
        const double e = (double)s_e[j] * exp(2.0 * ((double)s_mu[j] - (double)M));
        r = (float)(e / ((double)mi * (double)nj));
      }
      s_e[j] = r;
    }
  }
  __syncthreads();
  for (int j = tid; j < P; j += 256) {
    s_key[j] = (j < Ck && ko[j + 1] > ko[j]) ? desc_key(s_e[j], j) : ~0ull;
    if (srow && j < Ck) srow[j] = s_e[j];
  }
  __syncthreads();
  block_sort_keys(s_key, P);
  const double bud = row_budget ? (double)row_budget[(size_t)bh * Cq + i] : budget;
  // cumulative keys before each sorted position; each thread owns a run
  const int per = (P + 255) / 256;
  const int t0 = tid * per;
  int run = 0;
  for (int t = t0; t < min(P, t0 + per); ++t) {
    const uint64_t key = s_key[t];
    if (key != ~0ull) { const int jj = (int)(uint32_t)key; run += ko[jj + 1] - ko[jj]; }
  }
  int total;
  int before = block_exscan(run, s_scan, &total);
  for (int t = t0; t < min(P, t0 + per); ++t) {
    const uint64_t key = s_key[t];
    if (key == ~0ull) continue;
    const int jj = (int)(uint32_t)key;
    mrow[jj] = ((double)before < bud) ? 1 : 0;
    before += ko[jj + 1] - ko[jj];
  }
  // empty key clusters (sorted last with the all-ones key) are never taken
  for (int j = tid; j < Ck; j += 256)
    if (ko[j + 1] == ko[j]) mrow[j] = 0;
}

// ---------------------------------------------------------------- host side
struct RtPlan {
  int BH, Cqp, maxp;
  size_t off_qhi, off_qlo, off_sbar, off_ps, off_part, off_t1, off_bud, total;
};

static RtPlan rt_plan(int B, int H, int N, int D, int Cq, int Ck) {
  RtPlan p;
  p.BH = B * H;
  p.Cqp = round_up(Cq, 32);
  p.maxp = cdiv(N, RT_PIECE) + Ck;
  Carver cv(nullptr);
  p.off_qhi = cv.used; cv.take<bf16>((size_t)p.BH * p.Cqp * D);
  p.off_qlo = cv.used; cv.take<bf16>((size_t)p.BH * p.Cqp * D);
  p.off_sbar = cv.used; cv.take<float>((size_t)p.BH * Cq * Ck);
  p.off_ps = cv.used; cv.take<int32_t>((size_t)p.BH * (Ck + 1));
  p.off_part = cv.used; cv.take<float>((size_t)p.BH * p.maxp * Cq * 3);
  p.off_t1 = cv.used; cv.take<float>((size_t)p.BH * p.maxp);
  p.off_bud = cv.used; cv.take<int32_t>((size_t)p.BH * Cq);
  p.total = cv.used;
  return p;
}

static void launch_sbar(const float* q_means, const float* k_means, int BH, int Cq, int Ck, int D, float scale,
                        float* sbar, hipStream_t stream) {
  hipLaunchKernelGGL(rt_sbar_kernel, dim3(cdiv(Ck, 64), cdiv(Cq, 16), BH), dim3(256), 0, stream, q_means, k_means, Cq,
                     Ck, D, scale, sbar);
}

// The probe: q_bar hi/lo split, key pieces, per-(piece, query cluster) partial errors.
static void launch_probe(const RtPlan& p, const float* q_means, const void* k_perm, const void* v_perm, svgear_dtype dt,
                         const float* k_means, const float* v_means, const int32_t* k_offsets, int Cq, int Ck, int BH,
                         int N, int D, float scale, bf16* qh, bf16* ql, int32_t* ps, float* part, float* t1,
                         hipStream_t stream) {
  if (D == 128)
    hipLaunchKernelGGL((rt_prep_kernel<128>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       qh, ql);
  else
    hipLaunchKernelGGL((rt_prep_kernel<64>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       qh, ql);
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, k_offsets, Ck, RT_PIECE, ps);
#define RT_MAIN(T, DD)                                                                                              \
  hipLaunchKernelGGL((rt_main_kernel<T, DD>), dim3(p.maxp, BH), dim3(256), 0, stream, (const T*)k_perm,          \
                     (const T*)v_perm, k_means, v_means, k_offsets, ps, qh, ql, N, Cq, p.Cqp, Ck, p.maxp, scale, part, \
                     t1)
  if (dt == SVGEAR_BF16) {
    if (D == 128) RT_MAIN(bf16, 128); else RT_MAIN(bf16, 64);
  } else {
    if (D == 128) RT_MAIN(float, 128); else RT_MAIN(float, 64);
  }
#undef RT_MAIN
}

}  // namespace svg

using namespace svg;

extern "C" size_t svgear_route_workspace(int B, int H, int N, int D, int Cq, int Ck) {
  if (B < 1 || H < 1 || N < 1 || Cq < 1 || Ck < 1 || (D != 64 && D != 128)) return 0;
  return rt_plan(B, H, N, D, Cq, Ck).total;
}

extern "C" svgear_status svgear_route(const float* q_means, const int32_t* q_offsets, int Cq, const void* k_perm,
                                      const void* v_perm, svgear_dtype dt, const float* k_means, const float* v_means,
                                      const int32_t* k_offsets, int Ck, int B, int H, int N, int D, float scale,
                                      float density, const float* scores_in, float* scores_out, uint8_t* mask,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  svgear_status st = check_common("route", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (Cq < 1 || Cq > N || Cq > SVGEAR_MAX_CLUSTERS || Ck < 1 || Ck > N || Ck > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "route: Cq=%d, Ck=%d must be in [1, min(N=%d, %d)]", Cq, Ck, N,
                SVGEAR_MAX_CLUSTERS);
  if (!(scale > 0.f) || !(scale < INFINITY)) return fail(SVGEAR_ERR_INVALID_ARG, "route: scale must be > 0 and finite");
  if (!(density > 0.f && density <= 1.f)) return fail(SVGEAR_ERR_INVALID_ARG, "route: density must be in (0, 1]");
  if (!q_offsets || !k_offsets || !mask) return fail(SVGEAR_ERR_INVALID_ARG, "route: null pointer");
  if (!scores_in && (!q_means || !k_perm || !v_perm || !k_means || !v_means))
    return fail(SVGEAR_ERR_INVALID_ARG, "route: null pointer");
  RtPlan p = rt_plan(B, H, N, D, Cq, Ck);
  st = check_ws("route", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  bf16* qh = reinterpret_cast<bf16*>(w + p.off_qhi);
  bf16* ql = reinterpret_cast<bf16*>(w + p.off_qlo);
  float* sbar = reinterpret_cast<float*>(w + p.off_sbar);
  int32_t* ps = reinterpret_cast<int32_t*>(w + p.off_ps);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* t1 = reinterpret_cast<float*>(w + p.off_t1);
  const double budget = (double)density * (double)N;
  if (!scores_in) {
    launch_sbar(q_means, k_means, B * H, Cq, Ck, D, scale, sbar, stream);
    launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, B * H, N, D, scale, qh, ql, ps,
                 part, t1, stream);
  }
  hipLaunchKernelGGL(rt_select_kernel, dim3(Cq, B * H), dim3(256), 0, stream, part, t1, ps, sbar, q_offsets,
                     k_offsets, scores_in, Cq, Ck, p.maxp, budget, nullptr, scores_out, mask);
  return check_launch("svgear_route");
}

extern "C" svgear_status svgear_route_topp(const float* q_means, const int32_t* q_offsets, int Cq, const void* k_perm,
                                           const void* v_perm, svgear_dtype dt, const float* k_means,
                                           const float* v_means, const int32_t* k_offsets, int Ck, int B, int H, int N,
                                           int D, float scale, float top_p, int error_ranked, const float* probs_in,
                                           const float* scores_in, float* probs_out, float* scores_out,
                                           int32_t* budget_out, uint8_t* mask, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  svgear_status st = check_common("route_topp", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (Cq < 1 || Cq > N || Cq > SVGEAR_MAX_CLUSTERS || Ck < 1 || Ck > N || Ck > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: Cq=%d, Ck=%d must be in [1, min(N=%d, %d)]", Cq, Ck, N,
                SVGEAR_MAX_CLUSTERS);
  if (!(scale > 0.f) || !(scale < INFINITY))
    return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: scale must be > 0 and finite");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: top_p must be in (0, 1]");
  if (error_ranked != 0 && error_ranked != 1)
    return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: error_ranked must be 0 or 1");
  if (!error_ranked && (scores_in || scores_out))
    return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: ratios exist only with error_ranked = 1");
  if (!q_offsets || !k_offsets || !mask) return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: null pointer");
  const bool need_sbar = !probs_in || (error_ranked && !scores_in);
  const bool need_probe = error_ranked && !scores_in;
  if (need_sbar && (!q_means || !k_means)) return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: null pointer");
  if (need_probe && (!k_perm || !v_perm || !v_means)) return fail(SVGEAR_ERR_INVALID_ARG, "route_topp: null pointer");
  RtPlan p = rt_plan(B, H, N, D, Cq, Ck);
  st = check_ws("route_topp", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  char* w = static_cast<char*>(ws);
  bf16* qh = reinterpret_cast<bf16*>(w + p.off_qhi);
  bf16* ql = reinterpret_cast<bf16*>(w + p.off_qlo);
  float* sbar = reinterpret_cast<float*>(w + p.off_sbar);
  int32_t* ps = reinterpret_cast<int32_t*>(w + p.off_ps);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* t1 = reinterpret_cast<float*>(w + p.off_t1);
  int32_t* bud = budget_out ? budget_out : reinterpret_cast<int32_t*>(w + p.off_bud);
  const int BH = B * H;
  if (need_sbar) launch_sbar(q_means, k_means, BH, Cq, Ck, D, scale, sbar, stream);
  hipLaunchKernelGGL(rt_topp_kernel, dim3(Cq, BH), dim3(256), 0, stream, probs_in ? nullptr : sbar, probs_in,
                     q_offsets, k_offsets, Cq, Ck, (double)top_p, probs_out, bud, error_ranked ? nullptr : mask);
  if (error_ranked) {
    if (need_probe)
      launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, BH, N, D, scale, qh, ql, ps,
                   part, t1, stream);
    hipLaunchKernelGGL(rt_select_kernel, dim3(Cq, BH), dim3(256), 0, stream, part, t1, ps, sbar, q_offsets, k_offsets,
                       scores_in, Cq, Ck, p.maxp, 0.0, bud, scores_out, mask);
  }
  return check_launch("svgear_route_topp");
}
