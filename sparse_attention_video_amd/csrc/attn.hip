// Dynamic-block-size sparse attention with centroid compensation:
// svgear_sparse_attn.
//
// SVG2 summary, "Custom dynamic block-size sparse attention kernel": after the
// permutation every (query cluster, key cluster) block is a dense rectangle of
// any size, computed on the matrix cores without padding each block.  Here a
// workgroup takes up to 128 rows of one query cluster and streams the union of
// its selected key clusters as one packed sequence of 64-key tiles (clusters
// are contiguous in K'/V', so only the last tile of the whole stream is
// ragged), then the skipped non-empty clusters as pseudo-keys: key k_bar_j,
// value v_bar_j and a score raised by ln n_j (SVG-EAR: the skipped block's
// weight becomes n_j e^{q.k_bar_j / sqrt d}; FrontierCS blog toy example, task
// page walkthrough step 3).  Both parts share one online softmax (running max
// and sum in fp32), and each row is written back to its original position.
//
// MFMA formulation: S^T = K Q^T (keys x queries) and O^T = V^T P^T, so that a
// lane owns one query column of both, making the softmax statistics and the
// rescale of O lane-local.  bf16: QK^T and PV on v_mfma_f32_32x32x16_bf16,
// P rounded to bf16; the pseudo-keys' k_bar and v_bar (fp32) enter rounded to
// bf16 like the real keys and values.  fp32: v_mfma_f32_32x32x2f32
// throughout.
#include <float.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "host.h"
#include "scan.h"

namespace svg {

constexpr int AT_BM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int AT_BN = 64;   // keys per tile
constexpr int AT_REAL = 0, AT_PS = 1, AT_PSV = 2;  // tile kinds of the bf16 kernel

template <typename T, int D>
struct AttnLds {
  static constexpr bool F32 = sizeof(T) == 4;
  // bf16: K tiles [2][64][SK] (hi, lo) and V^T tiles [2][D][SV] (hi, lo)
  static constexpr int SK = F32 ? D + 1 : D + 8;
  static constexpr int SV = F32 ? D + 4 : AT_BN + 8;
  static constexpr size_t k_bytes = F32 ? (size_t)AT_BN * SK * 4 : (size_t)2 * AT_BN * SK * 2;
  static constexpr size_t v_bytes = F32 ? (size_t)AT_BN * SV * 4 : (size_t)2 * D * SV * 2;
  static constexpr size_t fixed = k_bytes + v_bytes + AT_BN * 4 /*bias*/ + 2 * AT_BN * 4 /*src*/;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) attn_kernel(const T* __restrict__ qp, const T* __restrict__ kp,
                                                   const T* __restrict__ vp, const int32_t* __restrict__ qidx,
                                                   const int32_t* __restrict__ qoff, const int32_t* __restrict__ tstart,
                                                   int Cq, const int32_t* __restrict__ koff, int Ck,
                                                   const float* __restrict__ kmeans, const float* __restrict__ vmeans,
                                                   const uint8_t* __restrict__ mask, int N, float sl2,
                                                   T* __restrict__ out, float* __restrict__ lse) {
  using L = AttnLds<T, D>;
  constexpr bool F32 = L::F32;
  constexpr int SK = L::SK, SV = L::SV;
  constexpr int KS = F32 ? D / 2 : D / 16;  // MFMA K-steps over the head dim
  constexpr int DT = D / 32;                // 32-wide output tiles over the head dim
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sK = smem;
  char* sV = smem + L::k_bytes;
  float* sBias = reinterpret_cast<float*>(sV + L::v_bytes);
  int* sSrc = reinterpret_cast<int*>(sBias + AT_BN);  // [2][64]
  int* sSelStart = sSrc + 2 * AT_BN;                  // [Ck]
  int* sSelPre = sSelStart + Ck;                      // [Ck + 1]
  int* sComp = sSelPre + Ck + 1;                      // [Ck]
  __shared__ int sScan[16];
  __shared__ int sInfo[4];

  const int bh = blockIdx.y, tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int half = lane >> 5, col = lane & 31;
  const int32_t* ts = tstart + (size_t)bh * (Cq + 1);
  if ((int)blockIdx.x >= ts[Cq]) return;
  block_upper_index(ts, Cq, blockIdx.x, &sInfo[0]);
  __syncthreads();
  const int ci = min(max(sInfo[0], 0), Cq - 1);  // (in range even for a malformed table)
  const int32_t* qo = qoff + (size_t)bh * (Cq + 1);
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int row0 = qo[ci] + ((int)blockIdx.x - ts[ci]) * AT_BM;
  const int rowEnd = qo[ci + 1];
  const uint8_t* mrow = mask + ((size_t)bh * Cq + ci) * Ck;

  // ---- compact the selected clusters (with key prefix) and the skipped non-empty ones
  {
    const int per = (Ck + 255) / 256;
    const int j0 = tid * per, j1 = min(Ck, j0 + per);
    int nsel = 0, ncomp = 0, nkeys = 0;
    for (int j = j0; j < j1; ++j) {
      const int nj = ko[j + 1] - ko[j];
      if (nj > 0) {
        if (mrow[j]) { ++nsel; nkeys += nj; } else { ++ncomp; }
      }
    }
    int tsel, tcomp, tkeys;
    int psel = block_exscan(nsel, sScan, &tsel);
    int pcomp = block_exscan(ncomp, sScan, &tcomp);
    int pkeys = block_exscan(nkeys, sScan, &tkeys);
    for (int j = j0; j < j1; ++j) {
      const int nj = ko[j + 1] - ko[j];
      if (nj > 0) {
        if (mrow[j]) {
          sSelStart[psel] = ko[j];
          sSelPre[psel] = pkeys;
          ++psel;
          pkeys += nj;
        } else {
          sComp[pcomp++] = j;
        }
      }
    }
    if (tid == 0) {
      sSelPre[tsel] = tkeys;
      sInfo[1] = tsel;
      sInfo[2] = tcomp;
      sInfo[3] = tkeys;
    }
    __syncthreads();
  }
  const int nsel = sInfo[1], ncomp = sInfo[2], nkeys = sInfo[3];
  const int nreal = (nkeys + AT_BN - 1) / AT_BN;
  const int ntiles = nreal + (ncomp + AT_BN - 1) / AT_BN;

  // ---- this wave's 32 query rows as MFMA B fragments (query = column)
  const T* qb = qp + (size_t)bh * N * D;
  const T* kb = kp + (size_t)bh * N * D;
  const T* vb = vp + (size_t)bh * N * D;
  const int qrow = row0 + 32 * w + col;
  const bool qok = qrow < rowEnd;
  bf16x8 bq[F32 ? 1 : KS];
  float bqf[F32 ? KS : 1];
  if constexpr (!F32) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (qok) v = *reinterpret_cast<const bf16x8*>(qb + (size_t)qrow * D + 16 * ks + 8 * half);
      bq[ks] = v;
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bqf[ks] = qok ? to_f32(qb[(size_t)qrow * D + 2 * ks + half]) : 0.f;
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  // source row (in K'/V') of stream position p of the selected keys
  auto src_of = [&](int p) -> int {
    if (p >= nkeys) return -1;
    const int s = upper_index(sSelPre, nsel, p);
    return sSelStart[s] + (p - sSelPre[s]);
  };
  if (tid < AT_BN && nreal > 0) sSrc[tid] = src_of(tid);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const bool pseudo = kt >= nreal;
    // ---- stage the tile: unit = (4 consecutive keys, 8 consecutive dims)
    {
      constexpr int UNITS = (AT_BN / 4) * (D / 8);
      for (int u = tid; u < UNITS; u += 256) {
        const int g4 = u / (D / 8), dc = u - g4 * (D / 8);
        const int d0 = dc * 8;
        float kf[4][8], vf[4][8];
        bool valid[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 4 * g4 + r;
          if (!pseudo) {
            const int src = sSrc[(kt & 1) * AT_BN + key];
            valid[r] = src >= 0;
            if constexpr (!F32) {
              bf16x8 kv = {}, vv = {};
              if (valid[r]) {
                kv = *reinterpret_cast<const bf16x8*>(kb + (size_t)src * D + d0);
                vv = *reinterpret_cast<const bf16x8*>(vb + (size_t)src * D + d0);
              }
#pragma unroll
              for (int e = 0; e < 8; ++e) { kf[r][e] = (float)kv[e]; vf[r][e] = (float)vv[e]; }
            } else {
              f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
              if (valid[r]) {
                k0 = *reinterpret_cast<const f32x4*>(kb + (size_t)src * D + d0);
                k1 = *reinterpret_cast<const f32x4*>(kb + (size_t)src * D + d0 + 4);
                v0 = *reinterpret_cast<const f32x4*>(vb + (size_t)src * D + d0);
                v1 = *reinterpret_cast<const f32x4*>(vb + (size_t)src * D + d0 + 4);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) { kf[r][e] = k0[e]; kf[r][e + 4] = k1[e]; vf[r][e] = v0[e]; vf[r][e + 4] = v1[e]; }
            }
          } else {
            const int c = (kt - nreal) * AT_BN + key;
            valid[r] = c < ncomp;
            f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
            if (valid[r]) {
              const int j = sComp[c];
              const float* kr = kmeans + ((size_t)bh * Ck + j) * D + d0;
              const float* vr = vmeans + ((size_t)bh * Ck + j) * D + d0;
              k0 = *reinterpret_cast<const f32x4*>(kr);
              k1 = *reinterpret_cast<const f32x4*>(kr + 4);
              v0 = *reinterpret_cast<const f32x4*>(vr);
              v1 = *reinterpret_cast<const f32x4*>(vr + 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) { kf[r][e] = k0[e]; kf[r][e + 4] = k1[e]; vf[r][e] = v0[e]; vf[r][e + 4] = v1[e]; }
            if (dc == 0) {
              float b = -INFINITY;
              if (valid[r]) {
                const int j = sComp[c];
                b = log2f((float)(ko[j + 1] - ko[j]));
              }
              sBias[key] = b;
            }
          }
          if (!pseudo && dc == 0) sBias[key] = valid[r] ? 0.f : -INFINITY;
        }
        if constexpr (!F32) {
          bf16* kh = reinterpret_cast<bf16*>(sK);
          bf16* kl = kh + AT_BN * SK;
          bf16* vh = reinterpret_cast<bf16*>(sV);
          bf16* vl = vh + D * SV;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16x8 h, l;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              bf16 hh, ll;
              split_bf16(kf[r][e], hh, ll);
              h[e] = hh;
              l[e] = ll;
            }
            *reinterpret_cast<bf16x8*>(&kh[(4 * g4 + r) * SK + d0]) = h;
            if (pseudo) *reinterpret_cast<bf16x8*>(&kl[(4 * g4 + r) * SK + d0]) = l;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bf16x4 h, l;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              bf16 hh, ll;
              split_bf16(vf[r][e], hh, ll);
              h[r] = hh;
              l[r] = ll;
            }
            *reinterpret_cast<bf16x4*>(&vh[(d0 + e) * SV + 4 * g4]) = h;
            if (pseudo) *reinterpret_cast<bf16x4*>(&vl[(d0 + e) * SV + 4 * g4]) = l;
          }
        } else {
          float* kf32 = reinterpret_cast<float*>(sK);
          float* vf32 = reinterpret_cast<float*>(sV);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kf32[(4 * g4 + r) * SK + d0 + e] = kf[r][e];
              vf32[(4 * g4 + r) * SV + d0 + e] = vf[r][e];
            }
        }
      }
      // next tile's sources
      if (kt + 1 < nreal && tid < AT_BN) sSrc[((kt + 1) & 1) * AT_BN + tid] = src_of((kt + 1) * AT_BN + tid);
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 acc = {};
      const int krow = sub * 32 + col;
      if constexpr (!F32) {
        const bf16* kh = reinterpret_cast<const bf16*>(sK);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kh[krow * SK + 16 * ks + 8 * half]);
          acc = mfma_bf16(a, bq[ks], acc);
        }
        if (pseudo) {
          const bf16* kl = kh + AT_BN * SK;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[krow * SK + 16 * ks + 8 * half]);
            acc = mfma_bf16(a, bq[ks], acc);
          }
        }
      } else {
        const float* kf32 = reinterpret_cast<const float*>(sK);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma_f32(kf32[krow * SK + 2 * ks + half], bqf[ks], acc);
      }
      s[sub] = acc;
    }

    // ---- online softmax (log2 domain); lane owns query `col`, 32 of the 64 keys
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float t = fmaf(s[sub][r], sl2, sBias[sub * 32 + c_row(r, half)]);
        s[sub][r] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[sub][r] - m_new);
        s[sub][r] = p;
        lsum += p;
      }
    l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (!F32) {
      const bf16* vh = reinterpret_cast<const bf16*>(sV);
      const bf16* vl = vh + D * SV;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int sub = st >> 1, tp = st & 1;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16)s[sub][8 * tp + e];
        const int k0 = 16 * st + 4 * half;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const int d = 32 * t + col;
          const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(&vh[d * SV + k0]);
          const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(&vh[d * SV + k0 + 8]);
          bf16x8 a;
#pragma unroll
          for (int e = 0; e < 4; ++e) { a[e] = x0[e]; a[e + 4] = x1[e]; }
          o[t] = mfma_bf16(a, pb, o[t]);
          if (pseudo) {
            const bf16x4 y0 = *reinterpret_cast<const bf16x4*>(&vl[d * SV + k0]);
            const bf16x4 y1 = *reinterpret_cast<const bf16x4*>(&vl[d * SV + k0 + 8]);
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) { b[e] = y0[e]; b[e + 4] = y1[e]; }
            o[t] = mfma_bf16(b, pb, o[t]);
          }
        }
      }
    } else {
      const float* vf32 = reinterpret_cast<const float*>(sV);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = sub * 32 + c_row(r, half);
#pragma unroll
          for (int t = 0; t < DT; ++t) o[t] = mfma_f32(vf32[key * SV + 32 * t + col], s[sub][r], o[t]);
        }
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, write rows back to their original positions
  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (qok) {
    const int orig = qidx[(size_t)bh * N + qrow];
    const float inv = 1.f / l_tot;
    T* orow = out + ((size_t)bh * N + orig) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * t + 8 * g + 4 * half;
        if constexpr (!F32) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[t][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + d) = v;
        } else {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[t][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(orow + d) = v;
        }
      }
    if (lse && half == 0) lse[(size_t)bh * N + orig] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------------------
// bf16 path.  Same algorithm, arranged for throughput on gfx950:
//  * K and V rows go straight from global memory into LDS
//    (buffer_load_dwordx4 ... lds, no registers); each lane follows the key
//    positions it loads with its own cursor over the selected-cluster list;
//  * the exposed cost inside a tile is LDS latency (the LDS itself is ~30%
//    busy), so K fragments are read two steps ahead of their products and
//    the V^T fragments of each 16-key step one step ahead, the order pinned
//    with scheduling groups;
//  * tiles are unpadded, 16-byte chunks swizzled per row (see below); the
//    S^T = K Q^T fragments are plain 16-byte reads, and the V^T fragments of
//    O^T = V^T P^T come from row-major V through the transposing LDS read
//    ds_read_b64_tr_b16;
//  * two tile buffers, each its own LDS array, so the reads of the tile in
//    use never wait for the loads of the next one;
//  * the running max is raised only when a tile's max exceeds it by more
//    than AT_LAZY (log2 units), so O and the sum are rarely rescaled (the
//    weights stay <= 2^AT_LAZY, and the final normalisation uses the same
//    max, so the result is unchanged);
//  * the row sum adds the bf16-rounded weights that multiply V (v_dot2), so
//    numerator and denominator use the same weights;
//  * skipped clusters (pseudo-keys: bf16 rows of the means, prepared once
//    per call) stream after the selected keys through the same loads.
//
// Tile layout: 64 rows of D bf16 (ROWB = 2 D bytes), chunk c (16 bytes) of
// row r in slot c ^ swz(r).  For D = 128 (64 LDS banks, 256 bytes per clock):
//   K: swz(r) = r & 15     -- 16 lanes of an A-fragment read touch 16
//                            consecutive rows at one chunk: 16 slots;
//   V: swz(r) = 4 (r & 3)  -- 32 lanes of a transposing read touch 4 rows x
//                            4 chunks: 16 slots.
// One load instruction fills 1 KiB = RPI consecutive rows; lane L writes
// slot L % CH of row L / CH (CH = chunks per row).
// ---------------------------------------------------------------------------
constexpr float AT_LAZY = 8.f;
constexpr int AT_XCDS = 8;  // MI355X: 8 XCDs, each with its own L2
// Largest one-dimensional grid of the bf16 kernel: 256-thread workgroups, at
// most 2^32 - 1 threads per launch, a multiple of AT_XCDS.
constexpr long long AT_MAX_GRID = ((4294967295LL / 256) / AT_XCDS) * AT_XCDS;

typedef __bf16 at_bf16x2 __attribute__((ext_vector_type(2)));
#define AT_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define AT_LDS16(p) ((__attribute__((address_space(3))) bf16x4*)(p))

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land
// at dst + 16 L (dst is the same for the whole wave).  The buffer form is
// counted on the vector-memory counter alone; the global (flat) form would
// also make every later LDS-read wait a full drain, which defeats reading
// fragments ahead.  Word 3 = 0x00020000: 32-bit data format, raw access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lds_src(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t src, uint32_t off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, AT_LDS(dst), 16, (int)off, 0, 0, 0);
}

// A fragment of V^T (8 keys at one dim) from two transposing reads of 4 keys each
__device__ __forceinline__ bf16x8 vt_frag(const char* p0, const char* p1) {
  const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(AT_LDS16(p0));
  const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(AT_LDS16(p1));
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// e4m3 products: A and B are 32 bytes per lane (row / column l % 32, k range
// 32 (l / 32) .. + 31 of the 64), fp32 accumulate; no block scaling
typedef int at_v8i __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_fp8(const at_v8i& a, const at_v8i& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// fp8 K tile: rows of D bytes, 16-byte chunks XOR-swizzled so that 16 rows
// read at one chunk fall on 16 different 4-bank groups
template <int D>
struct AtTile8 {
  static constexpr int ROWB = D, CH = D / 16, RPI = 64 / CH, NI = 16 / RPI, KK = D / 64;
  static __device__ __forceinline__ int swz(int r) { return (r / (256 / ROWB)) & (CH - 1); }
};

template <int D>
struct AtTile {
  static constexpr int ROWB = 2 * D, CH = D / 8, RPI = 64 / CH, NI = CH / 4;
  static constexpr int BYTES = AT_BN * ROWB;
  static __device__ __forceinline__ int swzK(int r) { return r & (CH >= 16 ? 15 : 7); }
  static __device__ __forceinline__ int swzV(int r) { return 4 * (r & (CH >= 16 ? 3 : 1)); }
};

// VAR: skipped clusters' scores also gain vcoef * sum_i q_i^2 Var_j[i]
// (variance-corrected compensation; vcoef in log2 units); the variances come
// in as bf16 rows of pkx (kvars itself is read by the operand preparation).
template <int D, bool VAR = false, bool F8 = false>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(const bf16* __restrict__ qp, const bf16* __restrict__ kp,
                                                           const bf16* __restrict__ vp, const int32_t* __restrict__ qidx,
                                                           const int32_t* __restrict__ qoff,
                                                           const int32_t* __restrict__ tstart, int Cq,
                                                           const int32_t* __restrict__ koff, int Ck,
                                                           const float* __restrict__ kmeans,
                                                           const float* __restrict__ vmeans,
                                                           const uint8_t* __restrict__ mask, int N, float sl2,
                                                           bf16* __restrict__ out, float* __restrict__ lse,
                                                           int maxt, int BHn, const float* __restrict__ kvars,
                                                           float vcoef, const int32_t* __restrict__ qexp,
                                                           const int32_t* __restrict__ kexp,
                                                           const bf16* __restrict__ pkx,
                                                           const bf16* __restrict__ pvx) {
  (void)kvars;
  using TL = AtTile<D>;
  using T8 = AtTile8<D>;
  constexpr int KS = D / 16, DT = D / 32, ROWB = TL::ROWB, CH = TL::CH, RPI = TL::RPI, NI = TL::NI;
  __shared__ __attribute__((aligned(1024))) char sK0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[TL::BYTES];
  __shared__ int sScan[16];
  __shared__ int sInfo[4];
  extern __shared__ __attribute__((aligned(16))) int sLists[];
  int* sSelStart = sLists;        // [Ck]  first permuted row of the c-th selected cluster
  int* sSelPre = sSelStart + Ck;  // [Ck+1] key position where the c-th selected cluster begins
  int* sComp = sSelPre + Ck + 1;  // [Ck]  skipped non-empty clusters
  // [Ck + 64] log2 n_j of the c-th skipped cluster (16-byte aligned)
  float* sPBias = reinterpret_cast<float*>(sLists + ((3 * Ck + 1 + 3) & ~3));

  // Workgroups are dealt to the 8 XCDs round-robin by linear id; give each XCD
  // a contiguous range of (head, tile) so the tiles of one query cluster, which
  // stream the same keys, run on the same XCD and share its L2.
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int half = lane >> 5, col = lane & 31;
  const int per_xcd = (int)gridDim.x / AT_XCDS;
  const int logical = ((int)blockIdx.x % AT_XCDS) * per_xcd + (int)blockIdx.x / AT_XCDS;
  const int bh = logical / maxt, tile = logical - bh * maxt;
  if (bh >= BHn) return;
  const int32_t* ts = tstart + (size_t)bh * (Cq + 1);
  if (tile >= ts[Cq]) return;
  block_upper_index(ts, Cq, tile, &sInfo[0]);
  __syncthreads();
  const int ci = min(max(sInfo[0], 0), Cq - 1);  // (in range even for a malformed table)
  const int32_t* qo = qoff + (size_t)bh * (Cq + 1);
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  const int row0 = qo[ci] + (tile - ts[ci]) * AT_BM;
  const int rowEnd = qo[ci + 1];
  const uint8_t* mrow = mask + ((size_t)bh * Cq + ci) * Ck;
  {
    const int per = (Ck + 255) / 256;
    const int j0 = tid * per, j1 = min(Ck, j0 + per);
    int nsel = 0, ncomp = 0, nkeys = 0;
    for (int j = j0; j < j1; ++j) {
      const int nj = ko[j + 1] - ko[j];
      if (nj > 0) {
        if (mrow[j]) { ++nsel; nkeys += nj; } else { ++ncomp; }
      }
    }
    int tsel, tcomp, tkeys;
    int psel = block_exscan(nsel, sScan, &tsel);
    int pcomp = block_exscan(ncomp, sScan, &tcomp);
    int pkeys = block_exscan(nkeys, sScan, &tkeys);
    for (int j = j0; j < j1; ++j) {
      const int nj = ko[j + 1] - ko[j];
      if (nj > 0) {
        if (mrow[j]) { sSelStart[psel] = ko[j]; sSelPre[psel] = pkeys; ++psel; pkeys += nj; }
        else { sComp[pcomp++] = j; }
      }
    }
    if (tid == 0) { sSelPre[tsel] = tkeys; sInfo[1] = tsel; sInfo[2] = tcomp; sInfo[3] = tkeys; }
    __syncthreads();
  }
  const int nsel = sInfo[1], ncomp = sInfo[2], nkeys = sInfo[3];
  const int nreal = (nkeys + AT_BN - 1) / AT_BN;

  // F8: qp and kp hold e4m3 bytes (D per row) with per-head power-of-two
  // scales 2^qexp, 2^kexp; real-tile scores use scale 2^(qexp+kexp) sl2 and
  // pseudo-tile scores (q against the fp32 means) 2^qexp sl2
  const bf16* qb = qp + (size_t)bh * N * D;
  const char* kb = F8 ? reinterpret_cast<const char*>(kp) + (size_t)bh * N * D
                      : reinterpret_cast<const char*>(kp + (size_t)bh * N * D);
  const char* q8b = reinterpret_cast<const char*>(qp) + (size_t)bh * N * D;
  const char* vb = reinterpret_cast<const char*>(vp + (size_t)bh * N * D);
  float sl2r = sl2, sl2p = sl2;
  if constexpr (F8) {
    sl2r = ldexpf(sl2, qexp[bh] + kexp[bh]);
    sl2p = ldexpf(sl2, qexp[bh]);
  }
  const int qrow = row0 + 32 * w + col;
  const bool qok = qrow < rowEnd;
  bf16x8 bq[KS];
  at_v8i bq8[F8 ? T8::KK : 1];
  if constexpr (!F8) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (qok) v = *reinterpret_cast<const bf16x8*>(qb + (size_t)qrow * D + 16 * ks + 8 * half);
      bq[ks] = v;
    }
  } else {
    // B operand of the e4m3 products: dims 64 kk + 32 half .. + 31 of the query row
#pragma unroll
    for (int kk = 0; kk < T8::KK; ++kk) {
      at_v8i v = {};
      if (qok) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(q8b + (size_t)qrow * D + 64 * kk + 32 * half);
        const u32x4 b = *reinterpret_cast<const u32x4*>(q8b + (size_t)qrow * D + 64 * kk + 32 * half + 16);
        v = at_v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      }
      bq8[kk] = v;
    }
  }
  // bf16 Q fragments from the e4m3 bytes (exact), for the pseudo tiles
  auto load_bq_from_fp8 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (qok) {
        const uint2 raw = *reinterpret_cast<const uint2*>(q8b + (size_t)qrow * D + 16 * ks + 8 * half);
        v[0] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.x, 0);
        v[1] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.x, 1);
        v[2] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.x, 2);
        v[3] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.x, 3);
        v[4] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.y, 0);
        v[5] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.y, 1);
        v[6] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.y, 2);
        v[7] = (bf16)__builtin_amdgcn_cvt_f32_fp8((int)raw.y, 3);
      }
      bq[ks] = v;
    }
  };
  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  // ---- per-lane LDS offsets
  // S^T A-fragment: row sub*32 + col, chunk 2 ks + half
  int aK[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aK[ks] = col * ROWB + (((2 * ks + half) ^ TL::swzK(col)) << 4);
  // V^T A-fragment by transposing reads: in each 16-lane group (j = lane % 16,
  // group g = lane / 16) lane j points at row kbase + j / 4, dims
  // 32 t + 16 (g & 1) + 4 (j % 4) .. +3; lane j then receives the 4 rows'
  // values at dim 32 t + 16 (g & 1) + j.
  int aV[DT];
  {
    const int j = lane & 15, g1 = (lane >> 4) & 1, r4 = j >> 2;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int chunk = 4 * t + 2 * g1 + ((j >> 1) & 1);
      aV[t] = (4 * half + r4) * ROWB + ((chunk ^ TL::swzV(r4)) << 4) + ((j & 1) << 3);
    }
  }
  // e4m3 K A-fragment: row sub*32 + col, chunks 4 kk + 2 half + {0, 1}
  int aK8[F8 ? T8::KK : 1][2];
  if constexpr (F8) {
#pragma unroll
    for (int kk = 0; kk < T8::KK; ++kk)
#pragma unroll
      for (int q = 0; q < 2; ++q) aK8[kk][q] = col * T8::ROWB + (((4 * kk + 2 * half + q) ^ T8::swz(col)) << 4);
  }
  // direct-to-LDS loads: instruction i of wave w fills rows (w NI + i) RPI + L / CH
  const int lq = lane / CH, lslot = lane % CH;
  int chK[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) chK[i] = lslot ^ TL::swzK((w * NI + i) * RPI + lq);
  const int chV = lslot ^ TL::swzV(lq);  // RPI is a multiple of 4

  // ---- source rows: each lane follows the key positions it loads,
  // kt * 64 + (w NI + i) RPI + lq, with its own cursor over the selected
  // clusters (positions only grow); positions past the end load row 0, whose
  // scores are masked
  int tc = 0, tc_base = nsel > 0 ? sSelStart[0] : 0, tc_pre = 0;
  int tc_nxt = nsel > 1 ? sSelPre[1] : 0x7fffffff;
  auto advance = [&](int p) {
    while (p >= tc_nxt) {
      ++tc;
      tc_base = sSelStart[tc];
      tc_pre = tc_nxt;
      tc_nxt = tc + 1 < nsel ? sSelPre[tc + 1] : 0x7fffffff;
    }
  };
  // the lane's rows are p0 + RPI i (i < NI); when every lane's rows lie in
  // one selected cluster before the end (a cluster boundary falls in the
  // wave's 16-row band of a tile about one time in ten) one cursor step and
  // one offset serve them all
  auto sources = [&](int kt, uint32_t* rowoff) {
    const int p0 = kt * AT_BN + w * NI * RPI + lq;
    const int pl = p0 + (NI - 1) * RPI;
    advance(p0);
    if (ballot(pl >= tc_nxt || pl >= nkeys) == 0) {
      const uint32_t r0 = (uint32_t)(tc_base + (p0 - tc_pre)) * (uint32_t)ROWB;
#pragma unroll
      for (int i = 0; i < NI; ++i) rowoff[i] = r0 + (uint32_t)(i * RPI * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int p = p0 + i * RPI;
        advance(p);
        rowoff[i] = (uint32_t)(p < nkeys ? tc_base + (p - tc_pre) : 0) * (uint32_t)ROWB;
      }
    }
  };
  // e4m3 K rows: instruction j of wave w fills rows (w NI8 + j) RPI8 + L / CH8
  // (the same 16-row band as the V rows of wave w), with a cursor of its own
  const int lq8 = lane / T8::CH, lslot8 = lane % T8::CH;
  int chK8[F8 ? T8::NI : 1];
  if constexpr (F8) {
#pragma unroll
    for (int j = 0; j < T8::NI; ++j) chK8[j] = lslot8 ^ T8::swz((w * T8::NI + j) * T8::RPI + lq8);
  }
  int uc = 0, uc_base = nsel > 0 ? sSelStart[0] : 0, uc_pre = 0;
  int uc_nxt = nsel > 1 ? sSelPre[1] : 0x7fffffff;
  auto sources8 = [&](int kt, uint32_t* rowoff) {
#pragma unroll
    for (int j = 0; j < (F8 ? T8::NI : 1); ++j) {
      const int p = kt * AT_BN + (w * T8::NI + j) * T8::RPI + lq8;
      while (p >= uc_nxt) {
        ++uc;
        uc_base = sSelStart[uc];
        uc_pre = uc_nxt;
        uc_nxt = uc + 1 < nsel ? sSelPre[uc + 1] : 0x7fffffff;
      }
      rowoff[j] = (uint32_t)(p < nkeys ? uc_base + (p - uc_pre) : 0) * (uint32_t)T8::ROWB;
    }
  };
  // a 32-bit per-lane offset from the head's base (4 address bytes per lane)
  // byte sizes of one head's rows: below 2^32 for N < 2^24 (checked on the host)
  const __amdgpu_buffer_rsrc_t rK = lds_src(kb, (uint32_t)N * (uint32_t)D * (F8 ? 1u : 2u));
  const __amdgpu_buffer_rsrc_t rV = lds_src(vb, (uint32_t)N * (uint32_t)D * 2u);
  auto issue = [&](const uint32_t* rowoff, const uint32_t* rowoff8, char* dK, char* dV) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int g = w * NI + i;
      if constexpr (!F8) load_lds16(rK, rowoff[i] + (uint32_t)(chK[i] << 4), dK + g * 1024);
      load_lds16(rV, rowoff[i] + (uint32_t)(chV << 4), dV + g * 1024);
    }
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < T8::NI; ++j)
        load_lds16(rK, rowoff8[j] + (uint32_t)(chK8[j] << 4), dK + (w * T8::NI + j) * 1024);
    }
  };

  // q^2 as bf16, the B operand of the variance products (variance variant)
  bf16x8 q2[VAR ? KS : 1];

  // one tile of keys in LDS: S^T, online softmax, O^T += V^T P^T.  Modes:
  //  AT_REAL  selected keys: the max is taken on the raw scores (scale > 0) and
  //           the scale folds into one FMA per weight;
  //  AT_PS    skipped clusters 64 pt .. 64 pt + 63 (rows of bf16 k_bar,
  //           v_bar): score q.k_bar scale + log2 n_j;
  //  AT_PSV   skipped clusters 32 pt .. 32 pt + 31, variance variant: K rows
  //           0..31 hold k_bar, rows 32..63 Var (multiplied by q^2), V rows
  //           0..31 v_bar: score q.k_bar scale + vcoef q^2.Var + log2 n_j.
  // All scores are in log2 units.
  auto compute = [&](const char* Kh, const char* Vh, int lim, auto mode_c, int pt, auto&& mid) {
    constexpr int mode = decltype(mode_c)::value;
    constexpr bool real = mode == AT_REAL, psv = mode == AT_PSV;
    constexpr int NST = psv ? 2 : 4;  // 16-key steps of O^T += V^T P^T
    f32x16 s[2] = {f32x16{}, f32x16{}};
    if constexpr (F8 && real) {
#pragma unroll
      for (int kk = 0; kk < T8::KK; ++kk)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const char* r = Kh + sub * 32 * T8::ROWB;
          const u32x4 a = *reinterpret_cast<const u32x4*>(r + aK8[kk][0]);
          const u32x4 b = *reinterpret_cast<const u32x4*>(r + aK8[kk][1]);
          const at_v8i fa = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
          s[sub] = mfma_fp8(fa, bq8[kk], s[sub]);
        }
    } else {
      // fragments of step ks + 2 are read before the products of step ks
      // (LDS latency exceeds the two products of one step)
      bf16x8 fr[3][2];
#pragma unroll
      for (int ks = 0; ks < 2 && ks < KS; ++ks) {
        fr[ks][0] = *reinterpret_cast<const bf16x8*>(Kh + aK[ks]);
        fr[ks][1] = *reinterpret_cast<const bf16x8*>(Kh + aK[ks] + 32 * ROWB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) {
          fr[(ks + 2) % 3][0] = *reinterpret_cast<const bf16x8*>(Kh + aK[ks + 2]);
          fr[(ks + 2) % 3][1] = *reinterpret_cast<const bf16x8*>(Kh + aK[ks + 2] + 32 * ROWB);
        }
        s[0] = mfma_bf16(fr[ks % 3][0], bq[ks], s[0]);
        s[1] = mfma_bf16(fr[ks % 3][1], psv ? q2[ks % (VAR ? KS : 1)] : bq[ks], s[1]);
      }
    }
    // V^T fragments of the first 16 keys: read now, used after the softmax
    bf16x8 vf[2][DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) vf[0][t] = vt_frag(Vh + aV[t], Vh + aV[t] + 8 * ROWB);
    mid();  // straight-line work that overlaps the products in flight
    if constexpr (!(F8 && real)) {
      // keep the read-ahead: the scheduler would otherwise sink each read to
      // just before its product; and spread the next tile's loads over the
      // products (one after each pair): issued as a burst they queue at the
      // texture unit, 1.3% slower (mask bits: 0x100 LDS read, 0x008 MFMA,
      // 0x020 vector-memory read)
      constexpr int LPK = (2 * NI + KS - 1) / KS;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, LPK, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 0);
    }
    if constexpr (mode == AT_PS) {
      // s[sub][r] = q.k_bar of skipped cluster 64 pt + sub*32 + c_row(r, half);
      // -inf past the last one
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 64 * pt + 32 * sub + 8 * g + 4 * half;
          const f32x4 b = *reinterpret_cast<const f32x4*>(sPBias + c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            s[sub][r] = c0 + e < ncomp ? fmaf(s[sub][r], sl2p, b[e]) : -INFINITY;
          }
        }
    } else if constexpr (psv) {
      // s[0][r] = q.k_bar and s[1][r] = q^2.Var of skipped cluster
      // 32 pt + c_row(r, half); -inf past the last one
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * pt + 8 * g + 4 * half;
        const f32x4 b = *reinterpret_cast<const f32x4*>(sPBias + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          s[0][r] = c0 + e < ncomp ? fmaf(s[0][r], sl2p, fmaf(s[1][r], vcoef, b[e])) : -INFINITY;
        }
      }
    } else if (lim < AT_BN) {
      // key index sub*32 + c_row(r, half) >= lim, with the lane's part moved to the right
      const int lh = lim - 4 * half;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (sub * 32 + 8 * (r >> 2) + (r & 3) >= lh) s[sub][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < (psv ? 1 : 2); ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    mx = max_halves(mx);
    if constexpr (real) mx *= sl2r;
    const bool grow = mx > m_run + AT_LAZY;
    if (ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }
    const float sc = real ? sl2r : 1.f;
    const float nm = -m_run;
    const at_bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int sub = st >> 1, tp = st & 1;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[sub][8 * tp + e], sc, nm));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const at_bf16x2 pr = {pb[2 * e], pb[2 * e + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
      }
      // the next 16 keys' fragments are read before these products
      if (st + 1 < NST) {
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const char* base = Vh + aV[t] + 16 * (st + 1) * ROWB;
          vf[(st + 1) & 1][t] = vt_frag(base, base + 8 * ROWB);
        }
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] = mfma_bf16(vf[st & 1][t], pb, o[t]);
    }
    // the next step's V^T reads go out before this step's products
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + 1 < NST) __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, DT, 1);
    }
  };
  using RealT = std::integral_constant<int, AT_REAL>;

  // ---- selected keys: packed 64-key tiles, double buffered, loop unrolled by
  // two so each half reads one fixed buffer
  if (nreal > 0) {
    uint32_t ro[NI], ro8[F8 ? T8::NI : 1];
    sources(0, ro);
    if constexpr (F8) sources8(0, ro8);
    issue(ro, ro8, sK0, sV0);
    // the Q fragments and tile 0 are in: later waits only cover the prefetch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nreal; kt += 2) {
      // the next tile's loads go out while this tile's S^T products run; past
      // the last tile they fetch row 0 into the idle buffer, which is never read
      sources(kt + 1, ro);
      if constexpr (F8) sources8(kt + 1, ro8);
      compute(sK0, sV0, nkeys - kt * AT_BN, RealT{}, 0, [&] { issue(ro, ro8, sK1, sV1); });
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kt + 1 < nreal) {
        sources(kt + 2, ro);
        if constexpr (F8) sources8(kt + 2, ro8);
        compute(sK1, sV1, nkeys - (kt + 1) * AT_BN, RealT{}, 0, [&] { issue(ro, ro8, sK0, sV0); });
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  }

  // ---- skipped non-empty clusters: pseudo-keys k_bar_j, v_bar_j, bias
  // log2 n_j, from bf16 rows prepared once per call, loaded straight into LDS
  // and double buffered like the real tiles: 64 clusters a tile, 32 with the
  // variance term (whose Var_j rows take the other half of the K tile)
  constexpr int PCL = VAR ? 32 : 64;
  const int npt = (ncomp + PCL - 1) / PCL;
  if (npt > 0) {
    if constexpr (F8) load_bq_from_fp8();
    if constexpr (VAR) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) q2[ks % (VAR ? KS : 1)][e] = (bf16)((float)bq[ks][e] * (float)bq[ks][e]);
    }
    for (int c = tid; c < ncomp; c += 256) {
      const int j = sComp[c];
      sPBias[c] = log2f((float)(ko[j + 1] - ko[j]));
    }
    constexpr int KROWS = VAR ? 2 : 1;  // K operand rows per cluster
    const __amdgpu_buffer_rsrc_t rPK = lds_src(
        reinterpret_cast<const char*>(pkx + (size_t)bh * Ck * KROWS * D), (uint32_t)(Ck * KROWS * D * 2));
    const __amdgpu_buffer_rsrc_t rPV =
        lds_src(reinterpret_cast<const char*>(pvx + (size_t)bh * Ck * D), (uint32_t)(Ck * D * 2));
    // rows of tile position p: K row KROWS j + part, V row j of skipped
    // cluster PCL pt + p % PCL (part = p / 32 with the variance term)
    auto psources = [&](int ptile, uint32_t* rk, uint32_t* rv) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int p = (w * NI + i) * RPI + lq;
        const int c = PCL * ptile + (p % PCL);
        const int j = c < ncomp ? sComp[c] : 0;
        rk[i] = (uint32_t)(KROWS * j + (VAR ? p / 32 : 0)) * (uint32_t)ROWB;
        rv[i] = (uint32_t)j * (uint32_t)ROWB;
      }
    };
    auto pissue = [&](const uint32_t* rk, const uint32_t* rv, char* dK, char* dV) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int g = w * NI + i;
        load_lds16(rPK, rk[i] + (uint32_t)(chK[i] << 4), dK + g * 1024);
        load_lds16(rPV, rv[i] + (uint32_t)(chV << 4), dV + g * 1024);
      }
    };
    using PsT = std::integral_constant<int, VAR ? AT_PSV : AT_PS>;
    uint32_t rk[NI], rv[NI];
    psources(0, rk, rv);
    pissue(rk, rv, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int pt = 0; pt < npt; pt += 2) {
      // past the last tile the loads fetch cluster 0's rows into the idle
      // buffer, which is never read
      psources(pt + 1, rk, rv);
      compute(sK0, sV0, AT_BN, PsT{}, pt, [&] { pissue(rk, rv, sK1, sV1); });
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (pt + 1 < npt) {
        psources(pt + 2, rk, rv);
        compute(sK1, sV1, AT_BN, PsT{}, pt + 1, [&] { pissue(rk, rv, sK0, sV0); });
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  }

  // ---- epilogue
  const float l_tot = sum_halves(l_run);
  if (qok) {
    const int orig = qidx[(size_t)bh * N + qrow];
    const float inv = 1.f / l_tot;
    bf16* orow = out + ((size_t)bh * N + orig) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[t][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * half) = v;
      }
    if (lse && half == 0) lse[(size_t)bh * N + orig] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  }
}
// ---------------------------------------------------------------- host side
struct AtPlan {
  int BH, maxt;
  size_t off_ts, off_pk, off_pv, total;
};

static AtPlan at_plan(int B, int H, int N, int D, int Cq, int Ck) {
  AtPlan p;
  p.BH = B * H;
  p.maxt = cdiv(N, AT_BM) + Cq;
  Carver cv(nullptr);
  p.off_ts = cv.used; cv.take<int32_t>((size_t)p.BH * (Cq + 1));
  p.off_pk = cv.used; cv.take<bf16>((size_t)p.BH * Ck * 2 * D);  // 2 rows per cluster with variances
  p.off_pv = cv.used; cv.take<bf16>((size_t)p.BH * Ck * D);
  p.total = cv.used;
  return p;
}

// pseudo-key operands of the bf16 kernel, rounded to bf16 (nearest even)
// like the rows of K'/V': pv row j = v_bar_j; pk row j = k_bar_j, or, with
// the variances (kvars non-null), pk rows 2j = k_bar_j and 2j + 1 = Var_j.
// Thread u converts 8 elements of one row.
__device__ __forceinline__ bf16x8 at_round8(const float* m) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(m);
  const f32x4 b = *reinterpret_cast<const f32x4*>(m + 4);
  bf16x8 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (bf16)a[e];
    h[e + 4] = (bf16)b[e];
  }
  return h;
}

template <int D>
__global__ void __launch_bounds__(256) at_pseudo_ops_kernel(const float* __restrict__ km,
                                                            const float* __restrict__ vm,
                                                            const float* __restrict__ kvars, int Ck,
                                                            bf16* __restrict__ pk, bf16* __restrict__ pv) {
  const int bh = blockIdx.y;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= Ck * (D / 8)) return;
  const int j = u / (D / 8), d0 = (u - j * (D / 8)) * 8;
  const size_t src = ((size_t)bh * Ck + j) * D + d0;
  *reinterpret_cast<bf16x8*>(pv + src) = at_round8(vm + src);
  if (kvars) {
    const size_t dst = ((size_t)bh * Ck + j) * 2 * D + d0;
    *reinterpret_cast<bf16x8*>(pk + dst) = at_round8(km + src);
    *reinterpret_cast<bf16x8*>(pk + dst + D) = at_round8(kvars + src);
  } else {
    *reinterpret_cast<bf16x8*>(pk + src) = at_round8(km + src);
  }
}

template <typename T, int D>
static void launch_attn(const void* q, const void* k, const void* v, const int32_t* qidx, const int32_t* qoff,
                        const int32_t* ts, int Cq, const int32_t* koff, int Ck, const float* km, const float* vm,
                        const uint8_t* mask, int BH, int N, float sl2, void* out, float* lse, int maxt,
                        const float* kvars, float vcoef, const int32_t* qexp, const int32_t* kexp,
                        const bf16* pk, const bf16* pv, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // cluster lists and the skipped clusters' biases; the tiles are static
    const size_t lds = (size_t)(((3 * Ck + 1 + 3) & ~3) + Ck + AT_BN) * sizeof(int);
    const int total = round_up(maxt * BH, AT_XCDS);
    if (kvars) {
      (void)hipFuncSetAttribute((const void*)attn_bf16_kernel<D, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
      hipLaunchKernelGGL((attn_bf16_kernel<D, true>), dim3(total), dim3(256), lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, qidx, qoff, ts, Cq, koff, Ck, km, vm, mask, N, sl2,
                         (bf16*)out, lse, maxt, BH, kvars, vcoef, (const int32_t*)nullptr,
                         (const int32_t*)nullptr, pk, pv);
    } else if (qexp) {
      (void)hipFuncSetAttribute((const void*)attn_bf16_kernel<D, false, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((attn_bf16_kernel<D, false, true>), dim3(total), dim3(256), lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, qidx, qoff, ts, Cq, koff, Ck, km, vm, mask, N, sl2,
                         (bf16*)out, lse, maxt, BH, (const float*)nullptr, 0.f, qexp, kexp, pk, pv);
    } else {
      (void)hipFuncSetAttribute((const void*)attn_bf16_kernel<D, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
      hipLaunchKernelGGL((attn_bf16_kernel<D, false>), dim3(total), dim3(256), lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, qidx, qoff, ts, Cq, koff, Ck, km, vm, mask, N, sl2,
                         (bf16*)out, lse, maxt, BH, (const float*)nullptr, 0.f, (const int32_t*)nullptr,
                         (const int32_t*)nullptr, pk, pv);
    }
  } else {
    (void)kvars;
    (void)vcoef;
    (void)qexp;
    (void)kexp;
    (void)pk;
    (void)pv;
    using L = AttnLds<T, D>;
    const size_t lds = L::fixed + (size_t)(3 * Ck + 1) * sizeof(int);
    (void)hipFuncSetAttribute((const void*)attn_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((attn_kernel<T, D>), dim3(maxt, BH), dim3(256), lds, st, (const T*)q, (const T*)k,
                       (const T*)v, qidx, qoff, ts, Cq, koff, Ck, km, vm, mask, N, sl2, (T*)out, lse);
  }
}

}  // namespace svg

using namespace svg;

// Whether one launch of the bf16 kernel can cover every (head, query tile).
static bool at_grid_fits(const AtPlan& p) { return (long long)p.maxt * p.BH + AT_XCDS <= AT_MAX_GRID; }

extern "C" size_t svgear_sparse_attn_workspace(int B, int H, int N, int D, int Cq, int Ck) {
  if (B < 1 || H < 1 || N < 1 || Cq < 1 || Ck < 1 || (D != 64 && D != 128)) return 0;
  if ((long long)B * H > 65535 || N >= (1 << 24)) return 0;
  const AtPlan p = at_plan(B, H, N, D, Cq, Ck);
  return at_grid_fits(p) ? p.total : 0;
}

// Every argument check of the attention calls (before anything is queued);
// fills the launch plan.
static svgear_status attn_check_args(const void* q_perm, const void* k_perm, const void* v_perm, svgear_dtype dt,
                                     const int32_t* q_perm_idx, const int32_t* q_offsets, int Cq,
                                     const int32_t* k_offsets, int Ck, const float* k_means, const float* v_means,
                                     const uint8_t* mask, int B, int H, int N, int D, float scale, void* out,
                                     AtPlan* plan) {
  svgear_status st = check_common("attn", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (Cq < 1 || Cq > N || Cq > SVGEAR_MAX_CLUSTERS || Ck < 1 || Ck > N || Ck > SVGEAR_MAX_CLUSTERS)
    return fail(SVGEAR_ERR_INVALID_ARG, "attn: Cq=%d, Ck=%d must be in [1, min(N=%d, %d)]", Cq, Ck, N,
                SVGEAR_MAX_CLUSTERS);
  if (!(scale > 0.f) || !(scale < INFINITY)) return fail(SVGEAR_ERR_INVALID_ARG, "attn: scale must be > 0 and finite");
  if (!q_perm || !k_perm || !v_perm || !q_perm_idx || !q_offsets || !k_offsets || !k_means || !v_means || !mask ||
      !out)
    return fail(SVGEAR_ERR_INVALID_ARG, "attn: null pointer");
  *plan = at_plan(B, H, N, D, Cq, Ck);
  if (!at_grid_fits(*plan))
    return fail(SVGEAR_ERR_INVALID_ARG, "attn: %lld query tiles exceed one launch's grid (B*H=%d, N=%d, Cq=%d)",
                (long long)plan->maxt * plan->BH, plan->BH, N, Cq);
  return SVGEAR_OK;
}

static svgear_status sparse_attn_impl(const void* q_perm, const void* k_perm, const void* v_perm, svgear_dtype dt,
                                      const int32_t* q_perm_idx, const int32_t* q_offsets, int Cq,
                                      const int32_t* k_offsets, int Ck, const float* k_means, const float* v_means,
                                      const float* k_vars, float strength, const uint8_t* mask, int B, int H, int N,
                                      int D, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                      hipStream_t stream, const int32_t* q_exp = nullptr,
                                      const int32_t* k_exp = nullptr) {
  AtPlan p;
  svgear_status st = attn_check_args(q_perm, k_perm, v_perm, dt, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means,
                                     v_means, mask, B, H, N, D, scale, out, &p);
  if (st != SVGEAR_OK) return st;
  st = check_ws("attn", ws, ws_bytes, p.total);
  if (st != SVGEAR_OK) return st;
  int32_t* ts = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.off_ts);
  const int BH = B * H;
  const float sl2 = scale * 1.4426950408889634f;
  // variance term in log2 units: strength * sigma^2 / 2 * log2(e), sigma^2 = scale^2 sum q_i^2 Var(k_i)
  const float vcoef = 0.5f * strength * scale * scale * 1.4426950408889634f;
  hipLaunchKernelGGL(chunk_list_kernel, dim3(BH), dim3(1024), 0, stream, q_offsets, Cq, AT_BM, ts);
  bf16* pk = reinterpret_cast<bf16*>(static_cast<char*>(ws) + p.off_pk);
  bf16* pv = reinterpret_cast<bf16*>(static_cast<char*>(ws) + p.off_pv);
  if (dt == SVGEAR_BF16) {
    const dim3 pg(cdiv(Ck * (D / 8), 256), BH);
    if (D == 128) {
      hipLaunchKernelGGL(at_pseudo_ops_kernel<128>, pg, dim3(256), 0, stream, k_means, v_means, k_vars, Ck, pk, pv);
      launch_attn<bf16, 128>(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, ts, Cq, k_offsets, Ck, k_means, v_means,
                             mask, BH, N, sl2, out, lse, p.maxt, k_vars, vcoef, q_exp, k_exp, pk, pv, stream);
    } else {
      hipLaunchKernelGGL(at_pseudo_ops_kernel<64>, pg, dim3(256), 0, stream, k_means, v_means, k_vars, Ck, pk, pv);
      launch_attn<bf16, 64>(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, ts, Cq, k_offsets, Ck, k_means, v_means,
                            mask, BH, N, sl2, out, lse, p.maxt, k_vars, vcoef, q_exp, k_exp, pk, pv, stream);
    }
  } else {
    if (D == 128)
      launch_attn<float, 128>(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, ts, Cq, k_offsets, Ck, k_means, v_means,
                              mask, BH, N, sl2, out, lse, p.maxt, k_vars, vcoef, q_exp, k_exp, pk, pv, stream);
    else
      launch_attn<float, 64>(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, ts, Cq, k_offsets, Ck, k_means, v_means,
                             mask, BH, N, sl2, out, lse, p.maxt, k_vars, vcoef, q_exp, k_exp, pk, pv, stream);
  }
  return check_launch("svgear_sparse_attn");
}

extern "C" svgear_status svgear_sparse_attn(const void* q_perm, const void* k_perm, const void* v_perm,
                                            svgear_dtype dt, const int32_t* q_perm_idx, const int32_t* q_offsets,
                                            int Cq, const int32_t* k_offsets, int Ck, const float* k_means,
                                            const float* v_means, const uint8_t* mask, int B, int H, int N, int D,
                                            float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  return sparse_attn_impl(q_perm, k_perm, v_perm, dt, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means, v_means,
                          nullptr, 0.f, mask, B, H, N, D, scale, out, lse, ws, ws_bytes, stream);
}

extern "C" svgear_status svgear_sparse_attn_var(const void* q_perm, const void* k_perm, const void* v_perm,
                                                svgear_dtype dt, const int32_t* q_perm_idx,
                                                const int32_t* q_offsets, int Cq, const int32_t* k_offsets, int Ck,
                                                const float* k_means, const float* v_means, const float* k_vars,
                                                float strength, const uint8_t* mask, int B, int H, int N, int D,
                                                float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
  if (dt != SVGEAR_BF16) return fail(SVGEAR_ERR_UNSUPPORTED, "attn_var: bf16 inputs only");
  if (!k_vars) return fail(SVGEAR_ERR_INVALID_ARG, "attn_var: null pointer");
  if (!(strength >= 0.f) || !(strength < INFINITY))
    return fail(SVGEAR_ERR_INVALID_ARG, "attn_var: strength must be >= 0 and finite");
  return sparse_attn_impl(q_perm, k_perm, v_perm, dt, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means, v_means,
                          k_vars, strength, mask, B, H, N, D, scale, out, lse, ws, ws_bytes, stream);
}

extern "C" svgear_status svgear_sparse_attn_fp8(const uint8_t* q8, const int32_t* q_exp, const uint8_t* k8,
                                                const int32_t* k_exp, const void* v_perm,
                                                const int32_t* q_perm_idx, const int32_t* q_offsets, int Cq,
                                                const int32_t* k_offsets, int Ck, const float* k_means,
                                                const float* v_means, const uint8_t* mask, int B, int H, int N,
                                                int D, float scale, void* out, float* lse, void* ws,
                                                size_t ws_bytes, hipStream_t stream) {
  if (!q_exp || !k_exp) return fail(SVGEAR_ERR_INVALID_ARG, "attn_fp8: null pointer");
  return sparse_attn_impl(q8, k8, v_perm, SVGEAR_BF16, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means, v_means,
                          nullptr, 0.f, mask, B, H, N, D, scale, out, lse, ws, ws_bytes, stream, q_exp, k_exp);
}

// ---------------------------------------------------------------- allocation-free variant
// Scratch of svgear_sparse_attn_noalloc: the tile list and the bf16
// pseudo-key rows of one call, in a static device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU reuses it (nothing in it needs to
// start at zero: each call writes all it reads), so calls that overlap on one
// GPU race.
static __device__ __attribute__((aligned(256))) unsigned char scratch[SVGEAR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int AT_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[AT_MAX_DEVICES] = {};
}  // namespace

// The device address of this GPU's copy of the scratch array.  In host code
// the array's name is only a stand-in, so the address is looked up once per
// device, with that device current, and kept.
static svgear_status noalloc_scratch(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(SVGEAR_ERR_HIP, "attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(SVGEAR_ERR_HIP, "attn_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= AT_MAX_DEVICES)
    return fail(SVGEAR_ERR_UNSUPPORTED, "attn_noalloc: device %d beyond the %d this build tracks", dev, AT_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(SVGEAR_ERR_HIP, "attn_noalloc: hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(SVGEAR_ERR_HIP, "attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SVGEAR_OK;
}

extern "C" svgear_status svgear_sparse_attn_noalloc(const void* q_perm, const void* k_perm, const void* v_perm,
                                                    svgear_dtype dt, const int32_t* q_perm_idx,
                                                    const int32_t* q_offsets, int Cq, const int32_t* k_offsets,
                                                    int Ck, const float* k_means, const float* v_means,
                                                    const uint8_t* mask, int B, int H, int N, int D, float scale,
                                                    void* out, float* lse, hipStream_t stream) {
  AtPlan p;
  svgear_status st = attn_check_args(q_perm, k_perm, v_perm, dt, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means,
                                     v_means, mask, B, H, N, D, scale, out, &p);
  if (st != SVGEAR_OK) return st;
  if (p.total > (size_t)SVGEAR_NOALLOC_SCRATCH_BYTES)
    return fail(SVGEAR_ERR_INVALID_ARG,
                "attn_noalloc: these sizes need %zu bytes of scratch, more than the library's %zu (use "
                "svgear_sparse_attn with a workspace)",
                p.total, (size_t)SVGEAR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = noalloc_scratch(stream, &ws);
  if (st != SVGEAR_OK) return st;
  return sparse_attn_impl(q_perm, k_perm, v_perm, dt, q_perm_idx, q_offsets, Cq, k_offsets, Ck, k_means, v_means,
                          nullptr, 0.f, mask, B, H, N, D, scale, out, lse, ws, (size_t)SVGEAR_NOALLOC_SCRATCH_BYTES,
                          stream);
}
