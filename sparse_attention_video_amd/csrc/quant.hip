// e4m3 quantisation of a [B, H, N, D] tensor with one power-of-two scale per
// (batch, head): svgear_quantize_fp8.
//
// SVG2 summary, results on HunyuanVideo: SVG2 combined with FP8 attention
// stacks with the sparsity (2.30x -> 2.55x end to end).  The pages give no
// scheme; here each (batch, head) slice gets the exponent e = the smallest
// integer with max|x| <= 448 * 2^e (448 = the largest finite e4m3 value), and
// code = e4m3(x * 2^-e) rounded to nearest even (OCP e4m3fn, the format of
// gfx950's conversion and matrix instructions), so x ~ code * 2^e.  A
// power-of-two scale keeps x * 2^-e exact, so the only rounding is the e4m3
// one.
#include <float.h>

#include "common.h"
#include "host.h"

namespace svg {

constexpr int QZ_THREADS = 256;
constexpr int QZ_VEC = 8;  // elements per thread per step

__global__ void qz_clear_kernel(uint32_t* __restrict__ amax, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[QZ_VEC]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < QZ_VEC; ++e) f[e] = (float)v[e];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[e + 4] = b[e]; }
  }
}

// max |x| per (batch, head); positive floats order like their bit patterns,
// so an integer atomic max is exact in any order
template <typename T>
__global__ void __launch_bounds__(QZ_THREADS) qz_amax_kernel(const T* __restrict__ x, size_t per_head,
                                                             uint32_t* __restrict__ amax) {
  __shared__ float s_m[QZ_THREADS / SV_WAVE];
  const int bh = blockIdx.y;
  const T* xb = x + (size_t)bh * per_head;
  float m = 0.f;
  for (size_t i = ((size_t)blockIdx.x * QZ_THREADS + threadIdx.x) * QZ_VEC; i < per_head;
       i += (size_t)gridDim.x * QZ_THREADS * QZ_VEC) {
    float f[QZ_VEC];
    load8(xb + i, f);
#pragma unroll
    for (int e = 0; e < QZ_VEC; ++e) m = fmaxf(m, fabsf(f[e]));
  }
  m = wave_max_f(m);
  if (lane_id() == 0) s_m[wave_id()] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = s_m[0];
    for (int i = 1; i < QZ_THREADS / SV_WAVE; ++i) b = fmaxf(b, s_m[i]);
    atomicMax(&amax[bh], __float_as_uint(b));
  }
}

// smallest e with a <= 448 * 2^e, from a = f 2^E (0.5 <= f < 1): 448 = 0.875 * 2^9
__device__ __forceinline__ int qz_exponent(float a) {
  if (!(a > 0.f)) return 0;
  int E;
  const float f = frexpf(a, &E);
  return f <= 0.875f ? E - 9 : E - 8;
}

template <typename T>
__global__ void __launch_bounds__(QZ_THREADS) qz_convert_kernel(const T* __restrict__ x, size_t per_head,
                                                                const uint32_t* __restrict__ amax,
                                                                uint8_t* __restrict__ x8, int32_t* __restrict__ exps) {
  const int bh = blockIdx.y;
  const int e = qz_exponent(__uint_as_float(amax[bh]));
  if (blockIdx.x == 0 && threadIdx.x == 0) exps[bh] = e;
  const T* xb = x + (size_t)bh * per_head;
  uint8_t* ob = x8 + (size_t)bh * per_head;
  for (size_t i = ((size_t)blockIdx.x * QZ_THREADS + threadIdx.x) * QZ_VEC; i < per_head;
       i += (size_t)gridDim.x * QZ_THREADS * QZ_VEC) {
    float f[QZ_VEC];
    load8(xb + i, f);
    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[0], -e), ldexpf(f[1], -e), lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[2], -e), ldexpf(f[3], -e), lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[4], -e), ldexpf(f[5], -e), hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[6], -e), ldexpf(f[7], -e), hi, true);
    *reinterpret_cast<uint2*>(ob + i) = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

}  // namespace svg

using namespace svg;

extern "C" size_t svgear_quantize_fp8_workspace(int B, int H) {
  if (B < 1 || H < 1) return 0;
  return align256((size_t)B * H * sizeof(uint32_t));
}

extern "C" svgear_status svgear_quantize_fp8(const void* x, svgear_dtype dt, int B, int H, int N, int D,
                                             uint8_t* x8, int32_t* exps, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  svgear_status st = check_common("quantize_fp8", dt, B, H, N, D);
  if (st != SVGEAR_OK) return st;
  if (!x || !x8 || !exps) return fail(SVGEAR_ERR_INVALID_ARG, "quantize_fp8: null pointer");
  st = check_ws("quantize_fp8", ws, ws_bytes, svgear_quantize_fp8_workspace(B, H));
  if (st != SVGEAR_OK) return st;
  const int BH = B * H;
  uint32_t* amax = static_cast<uint32_t*>(ws);
  const size_t per_head = (size_t)N * D;  // a multiple of QZ_VEC (D is 64 or 128)
  const size_t steps = (per_head + QZ_THREADS * QZ_VEC - 1) / (QZ_THREADS * QZ_VEC);
  const int blocks = (int)(steps < 64 ? steps : 64);
  hipLaunchKernelGGL(qz_clear_kernel, dim3(cdiv(BH, 256)), dim3(256), 0, stream, amax, BH);
  if (dt == SVGEAR_BF16) {
    hipLaunchKernelGGL(qz_amax_kernel<bf16>, dim3(blocks, BH), dim3(QZ_THREADS), 0, stream, (const bf16*)x, per_head,
                       amax);
    hipLaunchKernelGGL(qz_convert_kernel<bf16>, dim3(blocks, BH), dim3(QZ_THREADS), 0, stream, (const bf16*)x,
                       per_head, amax, x8, exps);
  } else {
    hipLaunchKernelGGL(qz_amax_kernel<float>, dim3(blocks, BH), dim3(QZ_THREADS), 0, stream, (const float*)x,
                       per_head, amax);
    hipLaunchKernelGGL(qz_convert_kernel<float>, dim3(blocks, BH), dim3(QZ_THREADS), 0, stream, (const float*)x,
                       per_head, amax, x8, exps);
  }
  return check_launch("svgear_quantize_fp8");
}
