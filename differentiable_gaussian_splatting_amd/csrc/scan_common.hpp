// Workgroup-wide exclusive prefix sum for wave64 workgroups (device helper shared by the sort and binning files).
#pragma once

#include <hip/hip_runtime.h>

namespace gsr {

// v from the lane the DPP control selects, 0 where the control selects no lane or the row mask disables the lane.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kCtrl, kRowMask, 0xF, true));
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_or_zero(uint64_t v) {
  return (uint64_t(dpp_or_zero<kCtrl, kRowMask>(uint32_t(v >> 32))) << 32) | dpp_or_zero<kCtrl, kRowMask>(uint32_t(v));
}

// Inclusive sum over the wave's lanes 0..lane, with DPP moves (no LDS round trips): row_shr 1, 2, 4, 8 within each
// 16-lane row, then row_bcast 15 (rows 1 and 3 add the last lane of the row before) and row_bcast 31 (rows 2 and 3
// add lane 31). All 64 lanes must be active.
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T x) {
  x += dpp_or_zero<0x111, 0xF>(x);
  x += dpp_or_zero<0x112, 0xF>(x);
  x += dpp_or_zero<0x114, 0xF>(x);
  x += dpp_or_zero<0x118, 0xF>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return x;
}

// Exclusive scan of one value per thread over a workgroup of kThreads (a multiple of 64) threads. `smem` holds
// kThreads / 64 elements. Every thread of the workgroup must call it. If total is non-null it receives the sum.
template <typename T, unsigned kThreads>
__device__ __forceinline__ T block_exclusive_scan(T v, T* total, T* smem) {
  constexpr unsigned kWaves = kThreads / 64;
  const unsigned lane = threadIdx.x & 63u, w = threadIdx.x / 64u;
  const T x = wave_inclusive_sum(v);
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

// Last-block-done without fences. Thread 0 of each of the nb blocks of a grid publishes its block's result with a
// device-scope atomic (an add or an exchange) and passes that atomic's return value here as `dep`. The count of
// finished blocks is then incremented at an address computed from `dep` (always `done`: `done_alias` is the same
// counter passed as a second argument, so the compiler cannot drop the choice), so the increment is issued only once
// the publishing atomic has returned, that is, has been performed where every block's atomics meet. Returns true
// for the block that counts last; it must read the published values with atomics (read-modify-write of 0), which
// then see every block's, and it returns the counter to 0 for the next launch. Device-scope fences would order the
// same accesses but write back the whole L2 of the issuing die in every block. No block waits for another.
__device__ __forceinline__ bool count_done_after(uint64_t dep, uint32_t* done, uint32_t* done_alias, uint32_t nb) {
  uint32_t* d = dep == ~uint64_t(0) ? done_alias : done;
  const uint32_t prev = atomicAdd(d, 1u);
  const bool last = prev == nb - 1;
  if (last) atomicExch(done, 0u);
  return last;
}

// The number of items a launch sized for `cap` items processes: cap itself, or with `dev` (a count that earlier
// launches on the stream computed on the device) *dev when it is at most cap, else none.
__device__ __forceinline__ uint64_t count_within(const uint64_t* dev, uint64_t cap) {
  if (!dev) return cap;
  const uint64_t v = *dev;
  return v <= cap ? v : 0;
}

// Lanes of this wave whose (valid) digit equals mine: one ballot per digit bit. Per bit, s is 0 or all ones (the
// bit, sign-extended), and the lanes that agree with mine are ~(ballot ^ s), formed on each 32-bit half: a bit
// extract, the ballot's compare, two XNORs and two ANDs.
template <uint32_t kBits>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
  const uint64_t v = __builtin_amdgcn_ballot_w64(valid);
  uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
#pragma unroll
  for (uint32_t bit = 0; bit < kBits; ++bit) {
    const uint32_t s = uint32_t(-int32_t((d >> bit) & 1u));
    const uint64_t b = __builtin_amdgcn_ballot_w64(s != 0u);
    lo &= ~(uint32_t(b) ^ s);
    hi &= ~(uint32_t(b >> 32) ^ s);
  }
  return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t lanemask_lt(uint32_t lane) { return (uint64_t(1) << lane) - 1; }

}  // namespace gsr
