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

#include <algorithm>
#include <type_traits>

namespace svg {

constexpr int RT_PIECE = 512;  // keys per workgroup piece
constexpr int RT_PROBE_PER_CU = 2;  // resident probe workgroups per compute unit (LDS-bound)
constexpr int RT_WAVES = 8;         // waves per probe workgroup, 16 query clusters each
constexpr int RT_PPW = 32;          // most pieces one probe workgroup streams
constexpr int SEL_MAX = SVGEAR_MAX_CLUSTERS;

// scale * log2(e) * q_bar split in bf16 hi/lo (the probe's products are then
// ds in log2 units), padded to a multiple of 32 rows with zeros.
template <int D>
__global__ void __launch_bounds__(256) rt_prep_kernel(const float* __restrict__ qm, int Cq, int Cqp, float scale2,
                                                      bf16* __restrict__ qhi, bf16* __restrict__ qlo) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= Cqp * D) return;
  const int row = i / D;
  const float v = row < Cq ? qm[(size_t)bh * Cq * D + i] * scale2 : 0.f;
  bf16 h, l;
  split_bf16(v, h, l);
  qhi[(size_t)bh * Cqp * D + i] = h;
  qlo[(size_t)bh * Cqp * D + i] = l;
}

// s_bar[i][j] = scale * q_bar_i . k_bar_j in fp64, rounded to fp32.  A block
// computes a 16 x 64 tile from rows staged in LDS (row stride D + 1 floats);
// every thread issues all its staging loads before storing any of them.
template <int D>
__global__ void __launch_bounds__(256) rt_sbar_kernel(const float* __restrict__ qm, const float* __restrict__ km,
                                                      int Cq, int Ck, float scale, float* __restrict__ sbar) {
  constexpr int S = D + 1;
  constexpr int NQ = 16 * D / 4 / 256, NK = 64 * D / 4 / 256;  // 16-byte loads per thread
  __shared__ float sq[16 * S];
  __shared__ float sk[64 * S];
  const int bh = blockIdx.z, i0 = blockIdx.y * 16, j0 = blockIdx.x * 64, tid = threadIdx.x;
  f32x4 vq[NQ], vk[NK];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int v = (tid + 256 * u) * 4, r = v / D;
    vq[u] = (i0 + r < Cq) ? *reinterpret_cast<const f32x4*>(qm + ((size_t)bh * Cq + i0) * D + v) : f32x4{};
  }
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int v = (tid + 256 * u) * 4, r = v / D;
    vk[u] = (j0 + r < Ck) ? *reinterpret_cast<const f32x4*>(km + ((size_t)bh * Ck + j0) * D + v) : f32x4{};
  }
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int v = (tid + 256 * u) * 4, r = v / D, d = v - r * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) sq[r * S + d + e] = vq[u][e];
  }
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int v = (tid + 256 * u) * 4, r = v / D, d = v - r * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) sk[r * S + d + e] = vk[u][e];
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

// Piece table: pieces are runs of <= RT_PIECE keys of one key cluster, in key
// order; piece pc of head bh is (cluster j, first key row r0, end row r1).
__global__ void __launch_bounds__(256) rt_pieces_kernel(const int32_t* __restrict__ koff,
                                                        const int32_t* __restrict__ pstart, int Ck, int maxp,
                                                        int4* __restrict__ pinfo) {
  const int bh = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Ck) return;
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
  const int lo = ko[j], hi = ko[j + 1];
  int4* out = pinfo + (size_t)bh * maxp;
  for (int pc = ps[j], r0 = lo; r0 < hi; ++pc, r0 += RT_PIECE) out[pc] = make_int4(j, r0, min(r0 + RT_PIECE, hi), 0);
}

// The probe.  A workgroup of RT_WAVES waves streams the pieces pc =
// blockIdx.x, blockIdx.x + gridDim.x, ... of one head, 32 keys (a sub-tile)
// at a time; wave w owns query clusters 16 (RT_WAVES pass + w) .. + 15, whose
// q_bar (hi and lo) it keeps in registers as the B operand of 16x16x32
// products.  Per sub-tile all threads (16 per key, D / 16 coordinates each)
// centre the keys on their cluster mean (k - k_bar, split hi/lo in bf16)
// into LDS, double buffered, together with the key's w_k = (v_bar -
// v_k).v_k and ||v_k||^2; each wave then takes the 3 hi/lo products of its
// queries against the sub-tile's two 16-key blocks (ds = scale q_bar.(k -
// k_bar), in log2 units) and folds them into its per-query (delta, S2, S3), which are
// lane-local (a lane owns one query column and 8 of the 32 keys).  At a
// piece's end the four lane groups of a query merge and go to part[(bh, pc,
// query)]; each wave's share of T1 = sum ||v_bar - v_k||^2 goes to
// t1part[(bh, pc, wave)].  Keys past a piece's end centre to zero rows and
// contribute nothing.
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// n elements of a row segment as floats (bf16 or fp32 source; n * sizeof(T)
// is 8, 16 or 32 bytes)
template <typename T, int n>
struct RtSeg {
  static constexpr int W = n * (int)sizeof(T) / 4;  // 32-bit words
  uint32_t v[W];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int u = 0; u < W; u += 4) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint32_t*>(p) + u);
        v[u] = x[0]; v[u + 1] = x[1]; v[u + 2] = x[2]; v[u + 3] = x[3];
      }
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      v[0] = x.x; v[1] = x.y;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int u = 0; u < W; ++u) v[u] = 0u;
  }
  __device__ __forceinline__ float at(int e) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = v[e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
      return __uint_as_float(v[e]);
    }
  }
};

template <typename T, int D>
__global__ void __launch_bounds__(RT_WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) rt_probe_kernel(
    const T* __restrict__ kp, const T* __restrict__ vp, const float* __restrict__ kmeans,
    const float* __restrict__ vmeans, const int4* __restrict__ pinfo, const int32_t* __restrict__ pstart,
    const bf16* __restrict__ qhi, const bf16* __restrict__ qlo, int N, int Cq, int Cqp, int Ck, int maxp,
    float* __restrict__ part, float* __restrict__ t1part) {
  constexpr int NT = RT_WAVES * 64;
  constexpr int KS = D / 32;   // 16x16x32 K-steps over the head dim
  constexpr int DPT = D / 16;  // coordinates per thread (16 threads per key)
  constexpr int SA = D + 8;    // LDS row stride (bf16) of the centred keys
  constexpr int QW = 16 * RT_WAVES;  // query clusters per pass
  constexpr int MSLOTS = RT_PPW * (2 * D / 4) / NT;  // 16-byte mean loads per thread in the prologue
  __shared__ __attribute__((aligned(16))) bf16 sA[2][2][32 * SA];  // [buffer][hi, lo][key row]
  __shared__ __attribute__((aligned(16))) float sW[2][32];
  __shared__ __attribute__((aligned(16))) float sVV[2][32];
  __shared__ __attribute__((aligned(16))) float sMean[RT_PPW][2 * D];  // k_bar | v_bar of each piece's cluster
  __shared__ float sVbsq[RT_PPW][16];  // ||v_bar||^2 over each thread segment
  __shared__ int4 sInfo[RT_PPW];
  __shared__ int2 sStream[RT_PPW * (RT_PIECE / 32)];  // (piece slot, first row) of each sub-tile
  __shared__ int sNsub;

  const int bh = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int grp = lane >> 4, col = lane & 15;
  const int kr = tid >> 4, seg = tid & 15, d0 = seg * DPT;  // key row in a sub-tile, coordinate segment
  const int P = pstart[(size_t)bh * (Ck + 1) + Ck];
  const int bx = blockIdx.x, G = gridDim.x;
  if (bx >= P) return;
  const int nall = (P - 1 - bx) / G + 1;  // pieces of this workgroup: bx, bx + G, ...
  const T* kb = kp + (size_t)bh * N * D;
  const T* vb = vp + (size_t)bh * N * D;

  // the pieces go in batches of RT_PPW: piece slot k of batch kb0 is piece
  // bx + (kb0 + k) G
  for (int kb0 = 0; kb0 < nall; kb0 += RT_PPW) {
  const int npc = min(RT_PPW, nall - kb0);
  // ---- prologue: piece table, cluster means and the sub-tile schedule in LDS
  if (tid < npc) sInfo[tid] = pinfo[(size_t)bh * maxp + bx + (kb0 + tid) * G];
  __syncthreads();
  {
    f32x4 mv[MSLOTS];
#pragma unroll
    for (int u = 0; u < MSLOTS; ++u) {
      const int v = tid + NT * u, k = v / (2 * D / 4), o = (v % (2 * D / 4)) * 4;
      mv[u] = f32x4{};
      if (k < npc) {
        const int j = sInfo[k].x;
        const float* src = o < D ? kmeans + ((size_t)bh * Ck + j) * D + o : vmeans + ((size_t)bh * Ck + j) * D + o - D;
        mv[u] = *reinterpret_cast<const f32x4*>(src);
      }
    }
#pragma unroll
    for (int u = 0; u < MSLOTS; ++u) {
      const int v = tid + NT * u, k = v / (2 * D / 4), o = (v % (2 * D / 4)) * 4;
      if (k < npc) *reinterpret_cast<f32x4*>(&sMean[k][o]) = mv[u];
    }
  }
  if (w == 0) {
    // exclusive scan of the pieces' sub-tile counts (RT_PPW <= 64 lanes)
    const int4 in = lane < npc ? sInfo[lane] : make_int4(0, 0, 0, 0);
    const int ns = lane < npc ? (in.z - in.y + 31) / 32 : 0;
    int x = ns;
#pragma unroll
    for (int o = 1; o < SV_WAVE; o <<= 1) {
      const int y = __shfl_up(x, o, SV_WAVE);
      if (lane >= o) x += y;
    }
    const int base = x - ns;
    for (int u = 0; u < ns; ++u) sStream[base + u] = make_int2(lane, in.y + 32 * u);
    if (lane == SV_WAVE - 1) sNsub = x;
  }
  __syncthreads();
  for (int u = tid; u < npc * 16; u += NT) {
    const int k = u >> 4, sg = u & 15;
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) t = fmaf(sMean[k][D + sg * DPT + e], sMean[k][D + sg * DPT + e], t);
    sVbsq[k][sg] = t;
  }
  __syncthreads();
  const int nsub = sNsub;

  // rows of sub-tile s for this thread (zeros past its piece's end)
  auto fetch = [&](int s, RtSeg<T, DPT>& rk, RtSeg<T, DPT>& rv) {
    bool ok = false;
    int r = 0;
    if (s < nsub) {
      const int2 st = sStream[s];
      r = st.y + kr;
      ok = r < sInfo[st.x].z;
    }
    if (ok) {
      rk.load(kb + (size_t)r * D + d0);
      rv.load(vb + (size_t)r * D + d0);
    } else {
      rk.zero();
      rv.zero();
    }
  };

  for (int qb = 0; qb < Cqp; qb += QW) {
    const int qt = qb / 16 + w;  // this wave's 16-query tile
    const bool has_q = qt * 16 < Cq;
    bf16x8 qh[KS], ql[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 h = {}, l = {};
      if (has_q) {
        const size_t o = ((size_t)bh * Cqp + qt * 16 + col) * D + 32 * ks + 8 * grp;
        h = *reinterpret_cast<const bf16x8*>(qhi + o);
        l = *reinterpret_cast<const bf16x8*>(qlo + o);
      }
      qh[ks] = h;
      ql[ks] = l;
    }
    RtSeg<T, DPT> rk[2], rv[2];
    fetch(0, rk[0], rv[0]);
    fetch(1, rk[1], rv[1]);
    float dl = 0.f, s2 = 0.f, s3 = 0.f, t1acc = 0.f;

    // one sub-tile: centre it into LDS[b] from register slot b, then fetch
    // sub-tile s + 2 into that slot, then the products and their statistics
    auto step = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
      const int2 st = sStream[s];
      const int k = st.x;
      {
        const bool ok = st.y + kr < sInfo[k].z;
        // per key: v_bar.v and ||v||^2 over this thread's coordinates; then
        // w = v_bar.v - ||v||^2 and ||v_bar - v||^2 = ||v_bar||^2 - 2 v_bar.v + ||v||^2
        float bvp = 0.f, vvp = 0.f;
        typedef __attribute__((__vector_size__(DPT * sizeof(__bf16)))) __bf16 bfv;
        bfv h = {}, l = {};
        if (ok) {
#pragma unroll
          for (int e0 = 0; e0 < DPT; e0 += 4) {
            const f32x4 kb4 = *reinterpret_cast<const f32x4*>(&sMean[k][d0 + e0]);
            const f32x4 vb4 = *reinterpret_cast<const f32x4*>(&sMean[k][D + d0 + e0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float kf = rk[b].at(e0 + e), vf = rv[b].at(e0 + e);
              const float dk = kf - kb4[e];
              const bf16 hh = (bf16)dk;
              h[e0 + e] = hh;
              l[e0 + e] = (bf16)(dk - (float)hh);
              bvp = fmaf(vb4[e], vf, bvp);
              vvp = fmaf(vf, vf, vvp);
            }
          }
        }
        *reinterpret_cast<bfv*>(&sA[b][0][kr * SA + d0]) = h;
        *reinterpret_cast<bfv*>(&sA[b][1][kr * SA + d0]) = l;
        if (ok) t1acc += sVbsq[k][seg] - 2.f * bvp + vvp;
        // the key's 16 threads are one 16-lane row of the wave (DPP sums)
        bvp = row16_sum(bvp);
        vvp = row16_sum(vvp);
        if (seg == 0) {
          sW[b][kr] = ok ? bvp - vvp : 0.f;
          sVV[b][kr] = ok ? vvp : 0.f;
        }
      }
      __syncthreads();
      fetch(s + 2, rk[b], rv[b]);
      // products of this wave's queries against the sub-tile's two 16-key
      // blocks: acc[h][j] is key 16 h + 4 grp + j for query col
      if (has_q) {
        f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const bf16* Ah = &sA[b][0][(16 * hb + col) * SA + 8 * grp];
          const bf16* Al = &sA[b][1][(16 * hb + col) * SA + 8 * grp];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Ah + 32 * ks);
            const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + 32 * ks);
            acc[hb] = mfma16_bf16(ah, qh[ks], acc[hb]);
            acc[hb] = mfma16_bf16(ah, ql[ks], acc[hb]);
            acc[hb] = mfma16_bf16(al, qh[ks], acc[hb]);
          }
        }
        float mx = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, acc[hb][j]);
        const float dn = fmaxf(dl, mx);
        if (dn > dl) {
          const float f = __builtin_amdgcn_exp2f(dl - dn);
          s2 *= f;
          s3 *= f * f;
          dl = dn;
        }
        const float a = __builtin_amdgcn_exp2f(-dn);
        float t2 = 0.f, t3 = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(&sW[b][16 * hb + 4 * grp]);
          const f32x4 vq = *reinterpret_cast<const f32x4*>(&sVV[b][16 * hb + 4 * grp]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float eps = __builtin_amdgcn_exp2f(acc[hb][j] - dn) - a;
            t2 = fmaf(eps, wv[j], t2);
            t3 = fmaf(eps * eps, vq[j], t3);
          }
        }
        s2 += t2;
        s3 += t3;
      }
      // a finished piece: merge the four lane groups of each query and write
      // its statistics
      if (s + 1 == nsub || sStream[s + 1].x != k) {
        const int pc = bx + (kb0 + k) * G;
        if (has_q) {
#pragma unroll
          for (int m = 16; m <= 32; m <<= 1) {
            const float od = shfl_xor(dl, m), o2 = shfl_xor(s2, m), o3 = shfl_xor(s3, m);
            const float dm = fmaxf(dl, od);
            const float fa = __builtin_amdgcn_exp2f(dl - dm), fb = __builtin_amdgcn_exp2f(od - dm);
            s2 = s2 * fa + o2 * fb;
            s3 = s3 * fa * fa + o3 * fb * fb;
            dl = dm;
          }
          const int q = qt * 16 + col;
          if (grp == 0 && q < Cq) {
            float* o = part + (((size_t)bh * maxp + pc) * Cq + q) * 3;
            o[0] = dl * 0.69314718055994531f;  // the stabiliser in natural-log units
            o[1] = s2;
            o[2] = s3;
          }
        }
        dl = 0.f;
        s2 = 0.f;
        s3 = 0.f;
        const float t1w = wave_sum_f(t1acc);
        if (qb == 0 && lane == 0) t1part[((size_t)bh * maxp + pc) * RT_WAVES + w] = t1w;
        t1acc = 0.f;
      }
    };
    for (int s = 0; s < nsub; s += 2) {
      step(s, std::integral_constant<int, 0>{});
      if (s + 1 < nsub) step(s + 1, std::integral_constant<int, 1>{});
    }
    __syncthreads();  // the next pass (or batch) rewrites the buffers and tables
  }
  }
}

// T1_j = sum over cluster j's keys of ||v_bar_j - v_k||^2, from the probe
// waves' shares, added in a fixed order (pieces ascending, waves ascending).
__global__ void __launch_bounds__(256) rt_t1_kernel(const float* __restrict__ t1part,
                                                    const int32_t* __restrict__ pstart, int Ck, int maxp,
                                                    float* __restrict__ t1c) {
  const int bh = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Ck) return;
  const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
  float T1 = 0.f;
  for (int pc = ps[j]; pc < ps[j + 1]; ++pc) {
    const float* t8 = t1part + ((size_t)bh * maxp + pc) * RT_WAVES;
    float tw = 0.f;
#pragma unroll
    for (int u = 0; u < RT_WAVES; ++u) tw += t8[u];
    T1 += tw;
  }
  t1c[(size_t)bh * Ck + j] = T1;
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
  // LDS sized to the call: P sort keys, Ck shares, Ck cluster sizes
  extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];
  int P = 1;
  while (P < Ck) P <<= 1;
  uint64_t* s_key = s_dyn;
  float* s_p = reinterpret_cast<float*>(s_key + P);
  int* s_n = reinterpret_cast<int*>(s_p + Ck);
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

__global__ void __launch_bounds__(256) rt_select_kernel(const float* __restrict__ part, const float* __restrict__ t1c,
                                                        const int32_t* __restrict__ pstart, const float* __restrict__ sbar,
                                                        const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
                                                        const float* __restrict__ scores_in, int Cq, int Ck, int maxp,
                                                        double budget, const int32_t* __restrict__ row_budget,
                                                        float* __restrict__ scores_out, uint8_t* __restrict__ mask) {
  // LDS sized to the call: P sort keys, Ck stabilised maxima, Ck errors / ratios
  extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];
  int P = 1;
  while (P < Ck) P <<= 1;
  uint64_t* s_key = s_dyn;
  float* s_mu = reinterpret_cast<float*>(s_key + P);
  float* s_e = s_mu + Ck;
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
  if (scores_in) {
    const float* in = scores_in + ((size_t)bh * Cq + i) * Ck;
    for (int j = tid; j < Ck; j += 256) s_e[j] = in[j];
  } else {
    const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
    float mloc = -INFINITY;
    for (int j = tid; j < Ck; j += 256) {
      float mu = -INFINITY, E = 0.f;
      if (ko[j + 1] > ko[j]) {
        // merge the cluster's pieces: up to 8 pieces' statistics are loaded
        // at once, then folded in piece order with rescaling to the running
        // stabiliser
        float dm = 0.f, S2 = 0.f, S3 = 0.f;
        for (int pc0 = ps[j]; pc0 < ps[j + 1]; pc0 += 8) {
          float o0[8], o1[8], o2[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool in = pc0 + u < ps[j + 1];
            const float* o = part + (((size_t)bh * maxp + (in ? pc0 + u : pc0)) * Cq + i) * 3;
            o0[u] = in ? o[0] : 0.f;
            o1[u] = in ? o[1] : 0.f;
            o2[u] = in ? o[2] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float dn = fmaxf(dm, o0[u]);
            const float fa = __expf(dm - dn), fb = __expf(o0[u] - dn);
            S2 = S2 * fa + o1[u] * fb;
            S3 = S3 * fa * fa + o2[u] * fb * fb;
            dm = dn;
          }
        }
        const float T1 = t1c[(size_t)bh * Ck + j];
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
  size_t off_qhi, off_qlo, off_sbar, off_ps, off_pinfo, off_part, off_t1, off_t1c, off_bud, total;
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
  p.off_pinfo = cv.used; cv.take<int4>((size_t)p.BH * p.maxp);
  p.off_part = cv.used; cv.take<float>((size_t)p.BH * p.maxp * Cq * 3);
  p.off_t1 = cv.used; cv.take<float>((size_t)p.BH * p.maxp * RT_WAVES);
  p.off_t1c = cv.used; cv.take<float>((size_t)p.BH * Ck);
  p.off_bud = cv.used; cv.take<int32_t>((size_t)p.BH * Cq);
  p.total = cv.used;
  return p;
}

// Dynamic LDS of the selection kernels: the sort keys of the next power of
// two >= Ck plus two Ck-long float (or int) tables.
static size_t sel_lds(int Ck) {
  int P = 1;
  while (P < Ck) P <<= 1;
  const size_t bytes = (size_t)P * 8 + (size_t)Ck * 8;
  (void)hipFuncSetAttribute((const void*)rt_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  (void)hipFuncSetAttribute((const void*)rt_topp_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return bytes;
}

static void launch_sbar(const float* q_means, const float* k_means, int BH, int Cq, int Ck, int D, float scale,
                        float* sbar, hipStream_t stream) {
  const dim3 grid(cdiv(Ck, 64), cdiv(Cq, 16), BH);
  if (D == 128)
    hipLaunchKernelGGL(rt_sbar_kernel<128>, grid, dim3(256), 0, stream, q_means, k_means, Cq, Ck, scale, sbar);
  else
    hipLaunchKernelGGL(rt_sbar_kernel<64>, grid, dim3(256), 0, stream, q_means, k_means, Cq, Ck, scale, sbar);
}

// The probe: q_bar hi/lo split, key pieces, per-(piece, query cluster) partial errors.
// Compute units of the current device (queried once per device).
static int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static void launch_probe(const RtPlan& p, const float* q_means, const void* k_perm, const void* v_perm, svgear_dtype dt,
                         const float* k_means, const float* v_means, const int32_t* k_offsets, int Cq, int Ck, int BH,
                         int N, int D, float scale, bf16* qh, bf16* ql, int32_t* ps, int4* pinfo, float* part,
                         float* t1, float* t1c, hipStream_t stream) {
  if (D == 128)
    hipLaunchKernelGGL((rt_prep_kernel<128>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       scale * 1.4426950408889634f, qh, ql);
  else
    hipLaunchKernelGGL((rt_prep_kernel<64>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       scale * 1.4426950408889634f, qh, ql);
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, k_offsets, Ck, RT_PIECE, ps);
  hipLaunchKernelGGL(rt_pieces_kernel, dim3(cdiv(Ck, 256), BH), dim3(256), 0, stream, k_offsets, ps, Ck, p.maxp,
                     pinfo);
  // workgroups per head: about RT_PROBE_WGS over the whole launch, each
  // streaming several pieces (never more workgroups than pieces can exist)
  // workgroups per head: about RT_PROBE_PER_CU per compute unit over the
  // whole launch (one round of resident workgroups), never more than pieces
  const int G = std::max(1, std::min(p.maxp, RT_PROBE_PER_CU * cu_count() / BH));
#define RT_PROBE(T, DD)                                                                                            \
  hipLaunchKernelGGL((rt_probe_kernel<T, DD>), dim3(G, BH), dim3(RT_WAVES * 64), 0, stream, (const T*)k_perm,              \
                     (const T*)v_perm, k_means, v_means, pinfo, ps, qh, ql, N, Cq, p.Cqp, Ck, p.maxp, part, t1)
  if (dt == SVGEAR_BF16) {
    if (D == 128) RT_PROBE(bf16, 128); else RT_PROBE(bf16, 64);
  } else {
    if (D == 128) RT_PROBE(float, 128); else RT_PROBE(float, 64);
  }
#undef RT_PROBE
  hipLaunchKernelGGL(rt_t1_kernel, dim3(cdiv(Ck, 256), BH), dim3(256), 0, stream, t1, ps, Ck, p.maxp, t1c);
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
  int4* pinfo = reinterpret_cast<int4*>(w + p.off_pinfo);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* t1 = reinterpret_cast<float*>(w + p.off_t1);
  float* t1c = reinterpret_cast<float*>(w + p.off_t1c);
  const double budget = (double)density * (double)N;
  if (!scores_in) {
    launch_sbar(q_means, k_means, B * H, Cq, Ck, D, scale, sbar, stream);
    launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, B * H, N, D, scale, qh, ql, ps,
                 pinfo, part, t1, t1c, stream);
  }
  hipLaunchKernelGGL(rt_select_kernel, dim3(Cq, B * H), dim3(256), sel_lds(Ck), stream, part, t1c, ps, sbar, q_offsets,
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
  int4* pinfo = reinterpret_cast<int4*>(w + p.off_pinfo);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* t1 = reinterpret_cast<float*>(w + p.off_t1);
  float* t1c = reinterpret_cast<float*>(w + p.off_t1c);
  int32_t* bud = budget_out ? budget_out : reinterpret_cast<int32_t*>(w + p.off_bud);
  const int BH = B * H;
  if (need_sbar) launch_sbar(q_means, k_means, BH, Cq, Ck, D, scale, sbar, stream);
  hipLaunchKernelGGL(rt_topp_kernel, dim3(Cq, BH), dim3(256), sel_lds(Ck), stream, probs_in ? nullptr : sbar, probs_in,
                     q_offsets, k_offsets, Cq, Ck, (double)top_p, probs_out, bud, error_ranked ? nullptr : mask);
  if (error_ranked) {
    if (need_probe)
      launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, BH, N, D, scale, qh, ql, ps,
                   pinfo, part, t1, t1c, stream);
    hipLaunchKernelGGL(rt_select_kernel, dim3(Cq, BH), dim3(256), sel_lds(Ck), stream, part, t1c, ps, sbar, q_offsets, k_offsets,
                       scores_in, Cq, Ck, p.maxp, 0.0, bud, scores_out, mask);
  }
  return check_launch("svgear_route_topp");
}
