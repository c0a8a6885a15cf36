// Workgroup-wide exclusive prefix sum for wave64 workgroups (device helper shared by the sort and binning files).
#pragma once

#include <hip/hip_runtime.h>

namespace gsr {

// Exclusive scan of one value per thread over a workgroup of kThreads (a multiple of 64) threads. `smem` holds
// kThreads / 64 elements. Every thread of the workgroup must call it. If total is non-null it receives the sum.
template <typename T, unsigned kThreads>
__device__ __forceinline__ T block_exclusive_scan(T v, T* total, T* smem) {
  constexpr unsigned kWaves = kThreads / 64;
  const unsigned lane = threadIdx.x & 63u, w = threadIdx.x / 64u;
  T x = v;
#pragma unroll
  for (unsigned off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) smem[w] = x;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (unsigned q = 0; q < kWaves; ++q) {
    const T s = smem[q];
    if (q < w) before += s;
    all += s;
  }
  __syncthreads();
  if (total) *total = all;
  return before + x - v;
}

}  // namespace gsr
