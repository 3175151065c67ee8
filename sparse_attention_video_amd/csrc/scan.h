// Block-wide integer scans and cluster chunk lists.
#pragma once

#include "common.h"

namespace svg {

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
// Returns the exclusive prefix of v; *total receives the block sum.
__device__ __forceinline__ int block_exscan(int v, int* smem /* >= 16 ints */, int* total) {
  const int lane = lane_id(), w = wave_id(), nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < SV_WAVE; o <<= 1) {
    int y = __shfl_up(x, o, SV_WAVE);
    if (lane >= o) x += y;
  }
  if (lane == SV_WAVE - 1) smem[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? smem[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(t, o, SV_WAVE);
      if (lane >= o) t += y;
    }
    if (lane < nw) smem[lane] = t;   // inclusive wave totals
  }
  __syncthreads();
  int base = w ? smem[w - 1] : 0;
  *total = smem[nw - 1];
  __syncthreads();
  return base + x - v;
}

// chunk_start[c] = sum_{c' < c} ceil(size(c') / rows); chunk_start[C] = total.
// One block (1024 threads) per (batch, head); each thread owns 4 clusters.
static __global__ void __launch_bounds__(1024) chunk_list_kernel(const int32_t* __restrict__ offsets, int C, int rows,
                                                          int32_t* __restrict__ chunk_start) {
  __shared__ int sm[16];
  const int bh = blockIdx.x;
  const int32_t* off = offsets + (size_t)bh * (C + 1);
  int32_t* cs = chunk_start + (size_t)bh * (C + 1);
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int c = threadIdx.x * 4 + e;
    int n = c < C ? off[c + 1] - off[c] : 0;
    loc[e] = (n + rows - 1) / rows;
    sum += loc[e];
  }
  int total;
  int base = block_exscan(sum, sm, &total);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int c = threadIdx.x * 4 + e;
    if (c < C) cs[c] = base;
    base += loc[e];
  }
  if (threadIdx.x == 0) cs[C] = total;
}

}  // namespace svg
