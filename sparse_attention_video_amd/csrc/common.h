// Device helpers shared by the SVG-EAR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/svgear.h"

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

#define SV_WAVE 64

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }  // round to nearest even

// Split v = hi + lo + r with hi, lo bfloat16 and |r| <= 2^-17 |v| (v - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(float v, bf16& hi, bf16& lo) {
  hi = (bf16)v;
  lo = (bf16)(v - (float)hi);
}

// ---------------------------------------------------------------- MFMA
// 32x32 output tiles.  Operand convention used throughout: lane l feeds A row
// (l % 32) and B column (l % 32); its 8 (bf16) or 1 (f32) elements occupy the
// K slots of group (l / 32).  The same (lane, element) -> K-slot map holds for
// A and B, so any consistent assignment of our own indices to (group, element)
// contracts correctly.  Output: lane l holds column (l % 32), rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int c_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (SV_WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, SV_WAVE); }

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  int2 p = *reinterpret_cast<int2*>(&v);
  p.x = __shfl_xor(p.x, m, SV_WAVE);
  p.y = __shfl_xor(p.y, m, SV_WAVE);
  return *reinterpret_cast<double*>(&p);
}

// Sum over the 64 lanes by a fixed butterfly (same order on every run).
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_d(v, m);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// max over lanes l and l ^ 32 (gfx950 v_permlane32_swap: no LDS round trip)
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Median of three floats (v_med3_f32).  Used on positive, finite keys whose
// float order equals their bit order.
__device__ __forceinline__ float med3f(float a, float b, float c) { return __builtin_amdgcn_fmed3f(a, b, c); }

// Sum over each row of 16 lanes by a fixed DPP butterfly (xor 1, xor 2,
// mirror within 8, mirror within 16); every lane of the row gets the same sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// The smaller of two positive, finite float keys, compared as bit patterns
// (an integer min: no NaN canonicalisation).
__device__ __forceinline__ float minkey(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

// Binary search: largest idx in [0, n) with starts[idx] <= v (starts[0] <= v assumed).
// Workgroup form for starts in global memory, with starts[0] <= v <
// starts[n]: exactly one i in [0, n) has starts[i] <= v < starts[i + 1]
// (the last i with starts[i] <= v), and the thread that tests it writes it
// to *out; every thread's loads are independent, so the lookup takes one
// memory latency instead of log2 n.  The caller synchronises before reading
// *out.
__device__ __forceinline__ void block_upper_index(const int32_t* starts, int n, int v, int* out) {
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (starts[i] <= v && starts[i + 1] > v) *out = i;
}

__device__ __forceinline__ int upper_index(const int32_t* starts, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 16-byte vector load/store helpers.
template <typename P>
__device__ __forceinline__ u32x4 ld16(const P* p) { return *reinterpret_cast<const u32x4*>(p); }
template <typename P>
__device__ __forceinline__ void st16(P* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
