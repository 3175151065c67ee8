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

// The probe for fp32 keys (bf16 keys take rt_probe_bf16_kernel below, which
// needs no centring).  A workgroup of RT_WAVES waves streams the pieces pc =
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

// Exact split v = hi + mid + lo into bfloat16 (v - hi and v - hi - mid are
// exact in fp32; the last remainder has at most 8 significant bits).
__device__ __forceinline__ void split3_bf16(float v, bf16& hi, bf16& mid, bf16& lo) {
  hi = (bf16)v;
  const float r1 = v - (float)hi;
  mid = (bf16)r1;
  lo = (bf16)(r1 - (float)mid);
}
// Two bf16 in a 32-bit word (element 0 in the low half), their doubles (exact),
// and a . b + c over the pair with exact products (v_dot2_f32_bf16).
__device__ __forceinline__ uint32_t pack_bf2(bf16 a, bf16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ uint32_t twice_bf2(uint32_t p) {
  const bf16 a = (bf16)(2.f * __uint_as_float(p << 16)), b = (bf16)(2.f * __uint_as_float(p & 0xFFFF0000u));
  return pack_bf2(a, b);
}
typedef __bf16 rt_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(rt_bf16x2, a), __builtin_bit_cast(rt_bf16x2, b), c, false);
}

// The probe for bfloat16 keys, without centring.  A bf16 key is exact, so the
// two 16x16x32 products of a key against the hi and lo planes of scale *
// log2(e) * q_bar give s_k = q2 . k (q2 = hi + lo, within 2^-17 of q_bar per
// coordinate) exact up to the fp32 accumulation.  A piece's reference score
// s'_j = q2 . k_bar_j is taken by the same product sequence on rows holding
// k_bar_j's exact three-piece bf16 split, summed, so that ds = s_k - s'_j =
// q2 . (k - k_bar_j) up to rounding (the centring kernel's ds carries the same
// 2^-17 truncation of q_bar), and a key equal to its cluster mean (a
// singleton, a cluster of identical members) gets ds = 0 exactly; the
// statistics are then those of rt_probe_kernel.  K sub-tiles go straight from
// global memory into two LDS tiles (each thread one 16-byte chunk, loads
// issued one sub-tile ahead; two separate arrays, so that the compiler's
// waits for an operand read cover only the tile it reads), rows past a
// piece's end repeat its last key, whose statistics are zeroed; the chunks of a row are XOR-swizzled so
// that the 16 rows of an operand read fall on distinct banks.  V rows come
// into registers for the per-key statistics as in rt_probe_kernel.
template <int D>
struct RtTile {
  static constexpr int ROWB = 2 * D, CH = D / 8, SLOTS = 32 * CH;  // 16-byte chunks per row, per sub-tile
  static __device__ __forceinline__ int swz(int r) { return CH == 16 ? (r & 15) : ((r >> 1) & 7); }
};

template <int D>
__global__ void __launch_bounds__(RT_WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) rt_probe_bf16_kernel(
    const bf16* __restrict__ kp, const bf16* __restrict__ vp, const float* __restrict__ kmeans,
    const float* __restrict__ vmeans, const int4* __restrict__ pinfo, const int32_t* __restrict__ pstart,
    const bf16* __restrict__ qhi, const bf16* __restrict__ qlo, int N, int Cq, int Cqp, int Ck, int maxp,
    float* __restrict__ part, float* __restrict__ t1part) {
  using TL = RtTile<D>;
  constexpr int NT = RT_WAVES * 64;
  constexpr int KS = D / 32;   // 16x16x32 K-steps over the head dim
  constexpr int DPT = D / 16;  // V coordinates per thread (16 threads per key)
  constexpr int QW = 16 * RT_WAVES;
  constexpr int MSLOTS = RT_PPW * (D / 4) / NT;  // 16-byte v_bar loads per thread in the prologue
  static_assert(TL::SLOTS <= NT && MSLOTS >= 1, "one K chunk per thread");
  __shared__ __attribute__((aligned(1024))) char sK0[32 * TL::ROWB];
  __shared__ __attribute__((aligned(1024))) char sK1[32 * TL::ROWB];
  // chunks of the waves beyond a sub-tile's (D = 64) land here, unused, so
  // that every thread issues the same loads and the load counts stay exact
  __shared__ __attribute__((aligned(1024))) char sKx[TL::SLOTS < NT ? 16 * (NT - TL::SLOTS) : 16];
  __shared__ __attribute__((aligned(16))) float sW[2][32];
  __shared__ __attribute__((aligned(16))) float sVV[2][32];
  // v_bar of each piece's cluster as an exact three-piece bf16 split (hi, mid,
  // lo planes of coordinate pairs), and ||v_bar||^2 over each thread segment
  __shared__ __attribute__((aligned(16))) uint32_t sVp[RT_PPW][3][D / 2];
  __shared__ float sVbsq[RT_PPW][16];
  __shared__ float sSb[RT_WAVES][RT_PPW][16];                    // s'_j of each piece, per wave query column
  __shared__ int4 sInfo[RT_PPW];
  // sub-tile s: (piece slot, first row, the piece's last row, 1 if the piece's last sub-tile)
  __shared__ int4 sStream[RT_PPW * (RT_PIECE / 32)];
  __shared__ int sNsub;

  const int bh = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int grp = lane >> 4, col = lane & 15;
  const int kr = tid >> 4, seg = tid & 15, d0 = seg * DPT;
  const int P = pstart[(size_t)bh * (Ck + 1) + Ck];
  const int bx = blockIdx.x, G = gridDim.x;
  if (bx >= P) return;
  const int nall = (P - 1 - bx) / G + 1;
  const bf16* kb = kp + (size_t)bh * N * D;
  const bf16* vb = vp + (size_t)bh * N * D;
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kb, (short)0, (int)((uint32_t)N * (uint32_t)TL::ROWB), 0x00020000);
  // this thread's K chunk in a sub-tile: row kq, chunk kc (stored at slot tid)
  const int kslot = tid % TL::SLOTS;
  const int kq = kslot / TL::CH, kc = (kslot % TL::CH) ^ TL::swz(kslot / TL::CH);

  for (int kb0 = 0; kb0 < nall; kb0 += RT_PPW) {
  const int npc = min(RT_PPW, nall - kb0);
  if (tid < npc) sInfo[tid] = pinfo[(size_t)bh * maxp + bx + (kb0 + tid) * G];
  __syncthreads();
  {
    f32x4 mv[MSLOTS];
#pragma unroll
    for (int u = 0; u < MSLOTS; ++u) {
      const int v = tid + NT * u, k = v / (D / 4), o = (v % (D / 4)) * 4;
      mv[u] = f32x4{};
      if (k < npc) mv[u] = *reinterpret_cast<const f32x4*>(vmeans + ((size_t)bh * Ck + sInfo[k].x) * D + o);
    }
#pragma unroll
    for (int u = 0; u < MSLOTS; ++u) {
      const int v = tid + NT * u, k = v / (D / 4), o = (v % (D / 4)) * 4;
      if (k < npc) {
        uint32_t pc[3][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16 a[3], c[3];
          split3_bf16(mv[u][2 * t], a[0], a[1], a[2]);
          split3_bf16(mv[u][2 * t + 1], c[0], c[1], c[2]);
#pragma unroll
          for (int pl = 0; pl < 3; ++pl) pc[pl][t] = pack_bf2(a[pl], c[pl]);
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) *reinterpret_cast<uint2*>(&sVp[k][pl][o / 2]) = make_uint2(pc[pl][0], pc[pl][1]);
      }
    }
  }
  if (w == 0) {
    const int4 in = lane < npc ? sInfo[lane] : make_int4(0, 0, 0, 0);
    const int ns = lane < npc ? (in.z - in.y + 31) / 32 : 0;
    int x = ns;
#pragma unroll
    for (int o = 1; o < SV_WAVE; o <<= 1) {
      const int y = __shfl_up(x, o, SV_WAVE);
      if (lane >= o) x += y;
    }
    const int base = x - ns;
    for (int u = 0; u < ns; ++u) sStream[base + u] = make_int4(lane, in.y + 32 * u, in.z - 1, u == ns - 1);
    if (lane == SV_WAVE - 1) sNsub = x;
  }
  __syncthreads();
  // ||v_bar||^2 = sum of hi^2 + 2 hi mid + 2 hi lo + mid^2 (the dropped terms
  // are below 2^-24 relative), in the pair order of the per-key products
  // below, so that for a v_bar exact in bf16 (mid = lo = 0) it repeats ||v||^2's
  // sequence of products exactly
  for (int u = tid; u < npc * 16; u += NT) {
    const int k = u >> 4, sg = u & 15;
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < DPT / 2; ++q) {
      const uint32_t h = sVp[k][0][sg * DPT / 2 + q], m = sVp[k][1][sg * DPT / 2 + q], l = sVp[k][2][sg * DPT / 2 + q];
      t = dot2_bf16(h, h, t);
      t = dot2_bf16(h, twice_bf2(m), t);
      t = dot2_bf16(h, twice_bf2(l), t);
      t = dot2_bf16(m, m, t);
    }
    sVbsq[k][sg] = t;
  }
  __syncthreads();
  const int nsub = sNsub;

  // K chunks of sub-tile s into tile kt, and this thread's V row segment of
  // sub-tile s.  Every thread always issues both loads (past the last
  // sub-tile, or past a piece's end, the rows are clamped to real ones whose
  // statistics are not used), so that the loads in flight are the same on
  // every path and the waits for them stay partial.
  auto kload = [&](int s, char* kt) {
    const int4 st = sStream[min(s, nsub - 1)];
    const int g = min(st.y + kq, st.z);
    char* dst = tid < TL::SLOTS ? kt + 1024 * w : sKx + 1024 * (w - TL::SLOTS / 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (__attribute__((address_space(3))) void*)dst, 16,
                                             (int)((uint32_t)g * TL::ROWB + kc * 16), 0, 0, 0);
  };
  auto fetch = [&](int s, RtSeg<bf16, DPT>& rv) {
    const int4 st = sStream[min(s, nsub - 1)];
    rv.load(vb + (size_t)min(st.y + kr, st.z) * D + d0);
  };

  for (int qb = 0; qb < Cqp; qb += QW) {
    const int qt = qb / 16 + w;
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
    // s_k for 16 rows whose K-step ks operand frag(ks) returns: the same
    // product sequence for keys and for the k_bar rows
    auto scores16 = [&](auto frag) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = frag(ks);
        acc = mfma16_bf16(a, qh[ks], acc);
        acc = mfma16_bf16(a, ql[ks], acc);
      }
      return acc;
    };
    if (has_q) {
      // s'_j: block bl holds pieces 4 bl + m in rows 4 m + t, t = 0, 1, 2 the
      // hi, mid, lo parts of k_bar (row 4 m + 3 zero); lane (col, grp) then
      // holds the three parts of piece 4 bl + grp for its query column
      for (int bl = 0; 4 * bl < npc; ++bl) {
        const int k = 4 * bl + (col >> 2), t = col & 3;
        const bool live = k < npc && t < 3;
        const float* src = kmeans + ((size_t)bh * Ck + (live ? sInfo[k].x : 0)) * D + 8 * grp;
        const f32x4 acc = scores16([&](int ks) {
          bf16x8 a = {};
          if (live) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + 32 * ks);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = e < 4 ? x0[e] : x1[e - 4];
              const bf16 h = (bf16)v;
              const float r1 = v - (float)h;
              const bf16 m = (bf16)r1;
              const bf16 l = (bf16)(r1 - (float)m);
              a[e] = t == 0 ? h : (t == 1 ? m : l);
            }
          }
          return a;
        });
        if (4 * bl + grp < npc) sSb[w][4 * bl + grp][col] = (acc[0] + acc[1]) + acc[2];
      }
    }
    RtSeg<bf16, DPT> rv[2];
    kload(0, sK0);
    fetch(0, rv[0]);
    __builtin_amdgcn_sched_barrier(0);  // keep sub-tile 0's load ahead of sub-tile 1's (the loop's waits count on it)
    fetch(1, rv[1]);
    __syncthreads();  // s'_j table written
    float dl = 0.f, s2 = 0.f, s3 = 0.f, t1acc = 0.f;

    auto step = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
      const int4 st = sStream[s];
      const int k = st.x;
      {
        const bool ok = st.y + kr <= st.z;
        float bvp = 0.f, vvp = 0.f;
        if (ok) {
          // v_bar . v and ||v||^2 from exact bf16 pair products: a key equal
          // to its (bf16-exact) mean gives bvp = vvp = ||v_bar||^2 bit for bit
          typedef __attribute__((__vector_size__(DPT * 2))) uint32_t pv_t;
          const pv_t hv = *reinterpret_cast<const pv_t*>(&sVp[k][0][d0 / 2]);
          const pv_t mv = *reinterpret_cast<const pv_t*>(&sVp[k][1][d0 / 2]);
          const pv_t lv = *reinterpret_cast<const pv_t*>(&sVp[k][2][d0 / 2]);
#pragma unroll
          for (int q = 0; q < DPT / 2; ++q) {
            const uint32_t v2 = rv[b].v[q];
            bvp = dot2_bf16(hv[q], v2, bvp);
            bvp = dot2_bf16(mv[q], v2, bvp);
            bvp = dot2_bf16(lv[q], v2, bvp);
            vvp = dot2_bf16(v2, v2, vvp);
          }
          t1acc += sVbsq[k][seg] - 2.f * bvp + vvp;
        }
        bvp = row16_sum(bvp);
        vvp = row16_sum(vvp);
        if (seg == 0) {
          sW[b][kr] = ok ? bvp - vvp : 0.f;
          sVV[b][kr] = ok ? vvp : 0.f;
        }
      }
      // this wave's K chunks of sub-tile s have landed (only the V load of
      // sub-tile s + 1 may still be in flight); after the barrier every
      // wave's have, and every wave is done with sub-tile s - 1's tile
      __builtin_amdgcn_s_waitcnt(0x0F71);
      __syncthreads();
      kload(s + 1, b ? sK0 : sK1);
      fetch(s + 2, rv[b]);
      if (has_q) {
        const char* kt = b ? sK1 : sK0;
        f32x4 acc[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int r = 16 * hb + col;
          acc[hb] = scores16([&](int ks) {
            return *reinterpret_cast<const bf16x8*>(kt + r * TL::ROWB + (((4 * ks + grp) ^ TL::swz(r)) << 4));
          });
        }
        const float sbp = sSb[w][k][col];
        float mx = acc[0][0];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, acc[hb][j]);
        const float dn = fmaxf(dl, mx - sbp);
        if (dn > dl) {
          const float f = __builtin_amdgcn_exp2f(dl - dn);
          s2 *= f;
          s3 *= f * f;
          dl = dn;
        }
        const float a = __builtin_amdgcn_exp2f(-dn);
        const float c = sbp + dn;
        float t2 = 0.f, t3 = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(&sW[b][16 * hb + 4 * grp]);
          const f32x4 vq = *reinterpret_cast<const f32x4*>(&sVV[b][16 * hb + 4 * grp]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float eps = __builtin_amdgcn_exp2f(acc[hb][j] - c) - a;
            t2 = fmaf(eps, wv[j], t2);
            t3 = fmaf(eps * eps, vq[j], t3);
          }
        }
        s2 += t2;
        s3 += t3;
      }
      if (st.w) {
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
            o[0] = dl * 0.69314718055994531f;
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
    // pairs of sub-tiles, then an odd last one (a loop that could also skip
    // its second step would merge load counts and make every wait a drain)
    int s = 0;
    for (; s + 1 < nsub; s += 2) {
      step(s, std::integral_constant<int, 0>{});
      step(s + 1, std::integral_constant<int, 1>{});
    }
    if (s < nsub) step(s, std::integral_constant<int, 0>{});
    __syncthreads();
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

// Error of key cluster j for query cluster i from the probe's per-piece
// statistics: the pieces are merged in piece order (up to 8 pieces' loads in
// flight at a time), each rescaled to the running stabiliser; E is the error
// relative to e^{2 mu} with mu = s_bar_ij + delta_ij (the cluster's largest
// probe score), i.e. e_ij = E e^{2 mu}.
__device__ __forceinline__ void cluster_error(const float* __restrict__ part, const float* __restrict__ t1c,
                                              const int32_t* __restrict__ ps, const float* __restrict__ sbar, int bh,
                                              int i, int j, int Cq, int Ck, int maxp, float& E, float& mu) {
  float dm = 0.f, S2 = 0.f, S3 = 0.f;
  const int pe = ps[j + 1];
  for (int pc0 = ps[j]; pc0 < pe; pc0 += 8) {
    float o0[8], o1[8], o2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = pc0 + u < pe;
      const float* o = part + (((size_t)bh * maxp + (in ? pc0 + u : pc0)) * Cq + i) * 3;
      o0[u] = in ? o[0] : 0.f;
      o1[u] = in ? o[1] : 0.f;
      o2[u] = in ? o[2] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (pc0 + u >= pe) break;  // (an absent piece would leave the sums unchanged)
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
}

// The ratio r_ij = e_ij e^{-2 M} / (|Q_i| |K_j|) from E and mu (M the row's
// largest mu), in fp64 and rounded once.
__device__ __forceinline__ float cluster_ratio(float E, float mu, float M, int mi, int nj) {
  const double e = (double)E * exp(2.0 * ((double)mu - (double)M));
  return (float)(e / ((double)mi * (double)nj));
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
        cluster_error(part, t1c, ps, sbar, bh, i, j, Cq, Ck, maxp, E, mu);
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
      s_e[j] = nj > 0 ? cluster_ratio(s_e[j], s_mu[j], M, mi, nj) : 0.f;
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

// Sum of an integer over the 16 lanes of each row (DPP butterfly, as
// row16_sum); every lane of the row gets its row's sum.
__device__ __forceinline__ int row16_sum_i(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);  // row_mirror
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v = row16_sum_i(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// The same selection with one wave per (batch, head, query cluster) when
// C_k <= 64 RT_SEL_CPL: cluster j = lane + 64 e lives in lane registers, and
// no sort is needed.  In the (r desc, j asc) order a cluster is taken while
// the keys of the clusters before it sum to less than the budget; the last
// one taken (the crossing cluster) is the one whose predecessors hold fewer
// than the budget's keys and which itself brings them to at least the
// budget.  Its sort key (the ratio part of desc_key, then j) is found bit by
// bit, each bit by one count over the wave of the keys of the clusters
// ordered before a candidate; every cluster ordered at or before it is taken.
constexpr int RT_SEL_CPL = 8;
constexpr int RT_SEL_JBITS = 9;  // bits of j < 64 RT_SEL_CPL
__global__ void __launch_bounds__(256) rt_select_wave_kernel(
    const float* __restrict__ part, const float* __restrict__ t1c, const int32_t* __restrict__ pstart,
    const float* __restrict__ sbar, const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
    const float* __restrict__ scores_in, int Cq, int Ck, int maxp, double budget,
    const int32_t* __restrict__ row_budget, float* __restrict__ scores_out, uint8_t* __restrict__ mask) {
  const int lane = lane_id();
  const int bh = blockIdx.y, i = blockIdx.x * 4 + wave_id();
  if (i >= Cq) return;  // whole waves; the kernel has no workgroup barrier
  const int32_t* qo = qoff + (size_t)bh * (Cq + 1);
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int mi = qo[i + 1] - qo[i];
  uint8_t* mrow = mask + ((size_t)bh * Cq + i) * Ck;
  float* srow = scores_out ? scores_out + ((size_t)bh * Cq + i) * Ck : nullptr;
  if (mi == 0) {
    for (int j = lane; j < Ck; j += SV_WAVE) {
      mrow[j] = 0;
      if (srow) srow[j] = 0.f;
    }
    return;
  }
  int nj[RT_SEL_CPL];
  float r[RT_SEL_CPL];
#pragma unroll
  for (int e = 0; e < RT_SEL_CPL; ++e) {
    const int j = lane + SV_WAVE * e;
    nj[e] = j < Ck ? ko[j + 1] - ko[j] : 0;
  }
  if (scores_in) {
    const float* in = scores_in + ((size_t)bh * Cq + i) * Ck;
#pragma unroll
    for (int e = 0; e < RT_SEL_CPL; ++e) {
      const int j = lane + SV_WAVE * e;
      r[e] = j < Ck ? in[j] : 0.f;
    }
  } else {
    const int32_t* ps = pstart + (size_t)bh * (Ck + 1);
    float E[RT_SEL_CPL], mu[RT_SEL_CPL], mloc = -INFINITY;
#pragma unroll
    for (int e = 0; e < RT_SEL_CPL; ++e) {
      E[e] = 0.f;
      mu[e] = -INFINITY;
      if (nj[e] > 0) {
        cluster_error(part, t1c, ps, sbar, bh, i, lane + SV_WAVE * e, Cq, Ck, maxp, E[e], mu[e]);
        mloc = fmaxf(mloc, mu[e]);
      }
    }
    const float M = wave_max_f(mloc);
#pragma unroll
    for (int e = 0; e < RT_SEL_CPL; ++e) r[e] = nj[e] > 0 ? cluster_ratio(E[e], mu[e], M, mi, nj[e]) : 0.f;
  }
  uint32_t kh[RT_SEL_CPL];  // ratio part of the sort key (empty clusters weigh nothing)
  int tot = 0;
#pragma unroll
  for (int e = 0; e < RT_SEL_CPL; ++e) {
    const int j = lane + SV_WAVE * e;
    if (srow && j < Ck) srow[j] = r[e];
    kh[e] = (uint32_t)(desc_key(r[e], j) >> 32);
    tot += nj[e];
  }
  tot = wave_sum_i(tot);
  const double bud = row_budget ? (double)row_budget[(size_t)bh * Cq + i] : budget;
  // a count of keys c is below the budget iff c < ceil(budget)
  const int cap = bud > (double)tot ? tot + 1 : (int)ceil(bud);
  uint32_t H = 0xFFFFFFFFu, L = 0xFFFFFFFFu;  // crossing cluster: all taken when every prefix is below the budget
  bool none = cap <= 0;
  if (!none && tot >= cap) {
    // H: the largest ratio key whose strictly smaller keys hold < cap keys
    H = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t c = H | (1u << b);
      int n = 0;
#pragma unroll
      for (int e = 0; e < RT_SEL_CPL; ++e) n += kh[e] < c ? nj[e] : 0;
      if (wave_sum_i(n) < cap) H = c;
    }
    int base = 0;
#pragma unroll
    for (int e = 0; e < RT_SEL_CPL; ++e) base += kh[e] < H ? nj[e] : 0;
    base = wave_sum_i(base);
    // L: among ratio key H, the largest j whose smaller indices hold < cap - base keys
    L = 0;
    for (int b = RT_SEL_JBITS - 1; b >= 0; --b) {
      const uint32_t c = L | (1u << b);
      int n = 0;
#pragma unroll
      for (int e = 0; e < RT_SEL_CPL; ++e) n += (kh[e] == H && (uint32_t)(lane + SV_WAVE * e) < c) ? nj[e] : 0;
      if (base + wave_sum_i(n) < cap) L = c;
    }
  }
#pragma unroll
  for (int e = 0; e < RT_SEL_CPL; ++e) {
    const int j = lane + SV_WAVE * e;
    if (j < Ck)
      mrow[j] = (!none && nj[e] > 0 && (kh[e] < H || (kh[e] == H && (uint32_t)j <= L))) ? 1 : 0;
  }
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

// The greedy fill: a wave per query cluster while the key clusters fit in its
// registers, else a workgroup per query cluster with a sort in LDS.
static void launch_select(const float* part, const float* t1c, const int32_t* ps, const float* sbar,
                          const int32_t* q_offsets, const int32_t* k_offsets, const float* scores_in, int Cq, int Ck,
                          int BH, int maxp, double budget, const int32_t* row_budget, float* scores_out,
                          uint8_t* mask, hipStream_t stream) {
  if (Ck <= SV_WAVE * RT_SEL_CPL)
    hipLaunchKernelGGL(rt_select_wave_kernel, dim3(cdiv(Cq, 4), BH), dim3(256), 0, stream, part, t1c, ps, sbar,
                       q_offsets, k_offsets, scores_in, Cq, Ck, maxp, budget, row_budget, scores_out, mask);
  else
    hipLaunchKernelGGL(rt_select_kernel, dim3(Cq, BH), dim3(256), sel_lds(Ck), stream, part, t1c, ps, sbar, q_offsets,
                       k_offsets, scores_in, Cq, Ck, maxp, budget, row_budget, scores_out, mask);
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
                         int N, int D, float scale, char* w, int32_t* ps, int4* pinfo, float* part, float* t1,
                         float* t1c, hipStream_t stream) {
  bf16* qh = reinterpret_cast<bf16*>(w + p.off_qhi);
  bf16* ql = reinterpret_cast<bf16*>(w + p.off_qlo);
  const float scale2 = scale * 1.4426950408889634f;
  if (D == 128)
    hipLaunchKernelGGL((rt_prep_kernel<128>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       scale2, qh, ql);
  else
    hipLaunchKernelGGL((rt_prep_kernel<64>), dim3(cdiv(p.Cqp * D, 256), BH), dim3(256), 0, stream, q_means, Cq, p.Cqp,
                       scale2, qh, ql);
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, k_offsets, Ck, RT_PIECE, ps);
  hipLaunchKernelGGL(rt_pieces_kernel, dim3(cdiv(Ck, 256), BH), dim3(256), 0, stream, k_offsets, ps, Ck, p.maxp,
                     pinfo);
  // workgroups per head: about RT_PROBE_PER_CU per compute unit over the
  // whole launch (one round of resident workgroups), never more than pieces
  const int G = std::max(1, std::min(p.maxp, RT_PROBE_PER_CU * cu_count() / BH));
  if (dt == SVGEAR_BF16) {
#define RT_PROBE(DD)                                                                                                 \
  hipLaunchKernelGGL((rt_probe_bf16_kernel<DD>), dim3(G, BH), dim3(RT_WAVES * 64), 0, stream, (const bf16*)k_perm,    \
                     (const bf16*)v_perm, k_means, v_means, pinfo, ps, qh, ql, N, Cq, p.Cqp, Ck, p.maxp, part, t1)
    if (D == 128) RT_PROBE(128); else RT_PROBE(64);
#undef RT_PROBE
  } else {
#define RT_PROBE(DD)                                                                                                 \
  hipLaunchKernelGGL((rt_probe_kernel<float, DD>), dim3(G, BH), dim3(RT_WAVES * 64), 0, stream, (const float*)k_perm, \
                     (const float*)v_perm, k_means, v_means, pinfo, ps, qh, ql, N, Cq, p.Cqp, Ck, p.maxp, part, t1)
    if (D == 128) RT_PROBE(128); else RT_PROBE(64);
#undef RT_PROBE
  }
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
  float* sbar = reinterpret_cast<float*>(w + p.off_sbar);
  int32_t* ps = reinterpret_cast<int32_t*>(w + p.off_ps);
  int4* pinfo = reinterpret_cast<int4*>(w + p.off_pinfo);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* t1 = reinterpret_cast<float*>(w + p.off_t1);
  float* t1c = reinterpret_cast<float*>(w + p.off_t1c);
  const double budget = (double)density * (double)N;
  if (!scores_in) {
    launch_sbar(q_means, k_means, B * H, Cq, Ck, D, scale, sbar, stream);
    launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, B * H, N, D, scale, w, ps,
                 pinfo, part, t1, t1c, stream);
  }
  launch_select(part, t1c, ps, sbar, q_offsets, k_offsets, scores_in, Cq, Ck, B * H, p.maxp, budget, nullptr,
                scores_out, mask, stream);
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
      launch_probe(p, q_means, k_perm, v_perm, dt, k_means, v_means, k_offsets, Cq, Ck, BH, N, D, scale, w, ps,
                   pinfo, part, t1, t1c, stream);
    launch_select(part, t1c, ps, sbar, q_offsets, k_offsets, scores_in, Cq, Ck, BH, p.maxp, 0.0, bud, scores_out, mask,
                  stream);
  }
  return check_launch("svgear_route_topp");
}
