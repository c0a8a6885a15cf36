// Binning: one (tile | depth) key per splat-tile overlap, a stable radix sort, per-tile ranges.
// [C0 resident arena + C1 pass skip page, section 2 table, rows "C0" and "C1"]
//
// Two orderings with bit-identical results:
//   GSR_BIN_KEY64   emit pairs splat by splat with key = (tile << 32) | depth bits, then sort the 64-bit keys
//                   (32 depth bits + the tile id's significant bits).
//   GSR_BIN_PRESORT sort the splats by depth bits first (n keys, not P), emit pairs in that order with the tile
//                   id as key, then sort by the tile id's significant bits only. A stable sort of the splats by
//                   (depth bits, index) followed by a stable sort of their pairs by tile gives each tile its pairs
//                   in (depth bits, splat index) order, which is exactly the stable order of the 64-bit keys.
// All extent arithmetic is one IEEE fp32 operation at a time (this file is compiled without contraction), with
// correctly rounded division and square root, so the rectangles equal a plain fp32 evaluation.
#include <algorithm>

#include "gsr_internal.hpp"
#include "scan_common.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kTileFirstAvg = 3072;  // the tile-first scheme's largest average list (its on-chip capacity: 3456)
constexpr uint32_t kScanItems = 16;
constexpr uint32_t kScanBlock = kThreads * kScanItems;

struct Rect {
  uint32_t tx0, ty0, w, h;  // w * h tiles; 0 when culled
};

// Validity test and the 3-sigma axis-aligned tile rectangle of one splat.
__device__ __forceinline__ Rect tile_rect(const float* __restrict__ sp, float depth, uint32_t tiles_x,
                                          uint32_t tiles_y) {
  const Rect none{0, 0, 0, 0};
  float v[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) v[k] = sp[k];
  bool finite = __builtin_isfinite(depth);
#pragma unroll
  for (int k = 0; k < 9; ++k) finite = finite && __builtin_isfinite(v[k]);
  if (!finite || !(depth > 0.0f)) return none;
  const float x = v[0], y = v[1], a = v[2], b = v[3], c = v[4], o = v[8];
  if (!(o >= 0.0f && o <= 1.0f) || !(a > 0.0f)) return none;
  const float ac = a * c;
  const float bb = b * b;
  const float det = ac - bb;
  if (!(det > 0.0f)) return none;
  const float rx = 3.0f * sqrtf(c / det);
  const float ry = 3.0f * sqrtf(a / det);
  const float fx0 = floorf((x - rx) / 16.0f);
  const float fx1 = floorf((x + rx) / 16.0f);
  const float fy0 = floorf((y - ry) / 16.0f);
  const float fy1 = floorf((y + ry) / 16.0f);
  const float cx0 = (0.0f < fx0) ? fx0 : 0.0f;
  const float mx = float(tiles_x - 1), my = float(tiles_y - 1);
  const float cx1 = (fx1 < mx) ? fx1 : mx;
  const float cy0 = (0.0f < fy0) ? fy0 : 0.0f;
  const float cy1 = (fy1 < my) ? fy1 : my;
  if (cx0 > cx1 || cy0 > cy1) return none;
  const uint32_t tx0 = uint32_t(cx0), ty0 = uint32_t(cy0);
  return Rect{tx0, ty0, uint32_t(cx1) - tx0 + 1, uint32_t(cy1) - ty0 + 1};
}

// Per splat, in index order (coalesced reads of the records): the tile rectangle and its tile count, the depth
// sort key and index for the presort scheme, and the block's count total in part[block].
// The exact-ellipse overlap rule (GSR_BIN_ELLIPSE): tile (tx, ty) of the box is kept when the 3-sigma ellipse
// (p - mean)^T [[a b][b c]] (p - mean) <= 9 meets the tile's closed square [16 tx, 16 tx + 16] x [16 ty, 16 ty + 16].
// The minimum of the quadratic over the square is 0 when the mean lies in it, else the least of the four edge
// minima (the vertex of the one-dimensional quadratic clamped to the edge). One IEEE fp32 operation at a time in
// this order, so the decision equals a plain fp32 evaluation of the same definition.
__device__ __forceinline__ float conic_q(float a, float b, float c, float dx, float dy) {
  return ((a * dx) * dx + ((b + b) * dx) * dy) + (c * dy) * dy;
}

__device__ __forceinline__ float clamp_f(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ __forceinline__ bool ellipse_meets_tile(float x, float y, float a, float b, float c, uint32_t tx,
                                                   uint32_t ty) {
  const float x0 = 16.0f * float(tx), x1 = x0 + 16.0f;
  const float y0 = 16.0f * float(ty), y1 = y0 + 16.0f;
  const float dx0 = x0 - x, dx1 = x1 - x;
  const float dy0 = y0 - y, dy1 = y1 - y;
  if (dx0 <= 0.0f && dx1 >= 0.0f && dy0 <= 0.0f && dy1 >= 0.0f) return true;
  float best = __builtin_huge_valf();
  float q = conic_q(a, b, c, dx0, clamp_f(-(b * dx0) / c, dy0, dy1));
  best = q < best ? q : best;
  q = conic_q(a, b, c, dx1, clamp_f(-(b * dx1) / c, dy0, dy1));
  best = q < best ? q : best;
  q = conic_q(a, b, c, clamp_f(-(b * dy0) / a, dx0, dx1), dy0);
  best = q < best ? q : best;
  q = conic_q(a, b, c, clamp_f(-(b * dy1) / a, dx0, dx1), dy1);
  best = q < best ? q : best;
  return best <= 9.0f;
}

// Number of the box's tiles the ellipse rule keeps.
__device__ uint32_t ellipse_count(const float* __restrict__ sp, const Rect& r) {
  const float x = sp[0], y = sp[1], a = sp[2], b = sp[3], c = sp[4];
  uint32_t cnt = 0;
  for (uint32_t dy = 0; dy < r.h; ++dy)
    for (uint32_t dx = 0; dx < r.w; ++dx) cnt += ellipse_meets_tile(x, y, a, b, c, r.tx0 + dx, r.ty0 + dy);
  return cnt;
}

// With dkeys, the depth sort's keys and values: the depth bits, and the splat index i, or with count_shift < 32
// i | count << count_shift (the presort scheme when both fit 32 bits), so that the sorted values carry the counts
// in depth order and the scan reads them in place instead of gathering them.
__global__ __launch_bounds__(kThreads) void k_prep(const float* __restrict__ splats, const float* __restrict__ depths,
                                                   uint32_t n, uint32_t tiles_x, uint32_t tiles_y, bool ellipse,
                                                   uint4* __restrict__ rects, uint32_t* __restrict__ counts,
                                                   uint32_t* __restrict__ dkeys, uint32_t* __restrict__ didx,
                                                   uint32_t count_shift, uint64_t* __restrict__ part) {
  __shared__ uint64_t smem[kThreads / kWave];
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  uint64_t c = 0;
  if (i < n) {
    const float depth = depths[i];
    const Rect r = tile_rect(splats + size_t(i) * 9, depth, tiles_x, tiles_y);
    rects[i] = make_uint4(r.tx0, r.ty0, r.w, r.h);
    c = ellipse ? ellipse_count(splats + size_t(i) * 9, r) : uint64_t(r.w) * r.h;
    counts[i] = uint32_t(c);
    if (dkeys) {
      dkeys[i] = __float_as_uint(depth);
      didx[i] = count_shift < 32 ? i | uint32_t(c) << count_shift : i;
    }
  }
  uint64_t total;
  block_exclusive_scan<uint64_t, kThreads>(c, &total, smem);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// *total = sum of part[0..nb), by one workgroup, also stored to the pinned host word *host_total, which the host
// reads once the launch has completed (one store instead of a copy launch). (A last-block-done sum inside k_prep
// would save this launch but serialise its 1,600 workgroups on one counter: 26 us against 6 + 5.)
__global__ __launch_bounds__(kThreads) void k_total(const uint64_t* __restrict__ part, uint32_t nb,
                                                    uint64_t* __restrict__ total, uint64_t* __restrict__ host_total) {
  __shared__ uint64_t smem[kThreads / kWave];
  uint64_t sum = 0;
  for (uint32_t j = threadIdx.x; j < nb; j += kThreads) sum += part[j];
  uint64_t all;
  block_exclusive_scan<uint64_t, kThreads>(sum, &all, smem);
  if (threadIdx.x == 0) {
    *total = all;
    *host_total = all;
  }
}

// Two-launch exclusive scan of uint32 counts into uint64 offsets; offsets[n] = total. With `order`, position j
// takes counts[order[j]] (order must be a permutation of 0..n-1; other entries count 0); without, counts[j] >> shift
// (shift 0: plain counts; else the depth-sorted values of k_prep, whose count field starts at bit shift).
__device__ __forceinline__ uint32_t count_at(const uint32_t* __restrict__ counts, const uint32_t* __restrict__ order,
                                             uint32_t n, uint64_t j, uint32_t shift) {
  if (!order) return counts[j] >> shift;
  const uint32_t i = order[j];
  return i < n ? counts[i] : 0u;
}

// Exclusive scan of part[0..nb) in place by one workgroup (reading the entries with atomics: see
// count_done_after); part[nb] and offsets[n] receive the total.
__device__ __forceinline__ void scan_parts(uint64_t* __restrict__ part, uint32_t nb, uint64_t* __restrict__ offsets,
                                           uint32_t n, uint64_t* smem) {
  uint64_t carry = 0;
  for (uint32_t c = 0; c < nb; c += kThreads) {
    const uint32_t j = c + threadIdx.x;
    const uint64_t v = j < nb ? atomicAdd(reinterpret_cast<unsigned long long*>(part + j), 0ull) : 0;
    uint64_t total;
    const uint64_t ex = block_exclusive_scan<uint64_t, kThreads>(v, &total, smem);
    if (j < nb) part[j] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    part[nb] = carry;
    offsets[n] = carry;
  }
}

// With `ordered`, the gathered counts are also stored in emission order for the down-sweep. Block sums are
// published with atomic exchanges; the block that finishes last reads them back with atomics, turns part[0..nb)
// into its exclusive scan and writes the total to part[nb] and offsets[n].
__global__ __launch_bounds__(kThreads) void k_scan_reduce(const uint32_t* __restrict__ counts,
                                                          const uint32_t* __restrict__ order, uint32_t shift,
                                                          uint32_t n,
                                                          uint64_t* __restrict__ part,
                                                          uint32_t* __restrict__ ordered, uint32_t* done,
                                                          uint32_t* done_alias, uint64_t* __restrict__ offsets) {
  __shared__ uint64_t smem[kThreads / kWave];
  __shared__ uint32_t s_last;
  const uint64_t base = uint64_t(blockIdx.x) * kScanBlock;
  uint64_t sum = 0;
  uint32_t c[kScanItems];
#pragma unroll
  for (uint32_t i = 0; i < kScanItems; ++i) {
    const uint64_t j = base + uint64_t(i) * kThreads + threadIdx.x;
    c[i] = j < n ? count_at(counts, order, n, j, shift) : 0u;
  }
#pragma unroll
  for (uint32_t i = 0; i < kScanItems; ++i) {
    const uint64_t j = base + uint64_t(i) * kThreads + threadIdx.x;
    sum += c[i];
    if (ordered && j < n) ordered[j] = c[i];
  }
  uint64_t total;
  block_exclusive_scan<uint64_t, kThreads>(sum, &total, smem);
  if (threadIdx.x == 0) {
    const uint64_t before = atomicExch(reinterpret_cast<unsigned long long*>(part + blockIdx.x), total);
    s_last = count_done_after(before, done, done_alias, gridDim.x) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  scan_parts(part, gridDim.x, offsets, n, smem);
}

__global__ __launch_bounds__(kThreads) void k_scan_down(const uint32_t* __restrict__ counts,
                                                        const uint32_t* __restrict__ order, uint32_t shift,
                                                        uint32_t n,
                                                        const uint64_t* __restrict__ part,
                                                        uint64_t* __restrict__ offsets) {
  __shared__ uint64_t smem[kThreads / kWave];
  const uint64_t base = uint64_t(blockIdx.x) * kScanBlock + uint64_t(threadIdx.x) * kScanItems;
  uint32_t c[kScanItems];
  uint64_t sum = 0;
#pragma unroll
  for (uint32_t i = 0; i < kScanItems; ++i) {
    c[i] = (base + i < n) ? count_at(counts, order, n, base + i, shift) : 0u;
    sum += c[i];
  }
  uint64_t run = part[blockIdx.x] + block_exclusive_scan<uint64_t, kThreads>(sum, nullptr, smem);
#pragma unroll
  for (uint32_t i = 0; i < kScanItems; ++i) {
    if (base + i < n) offsets[base + i] = run;
    run += c[i];
  }
}

// k / w for k < 2^20 and w >= 1 by a float quotient (the fast reciprocal is within 2^-22 relative, so the
// truncated quotient is off by at most one) and one correction; larger k take the integer division.
__device__ __forceinline__ uint32_t div_small(uint32_t k, uint32_t w) {
  if (k >= (1u << 20)) return k / w;
  uint32_t q = uint32_t(float(k) * __builtin_amdgcn_rcpf(float(w)));
  const int32_t r = int32_t(k) - int32_t(q * w);
  if (r < 0)
    --q;
  else if (r >= int32_t(w))
    ++q;
  return q;
}

// Exclusive running maximum over a workgroup of kThreads threads (a multiple of 64), seeded with `carry`: thread t
// gets the maximum of carry and the values of threads 0..t-1. Every thread must call it. `total` receives the
// maximum over the workgroup and the carry.
template <unsigned kThreads>
__device__ __forceinline__ uint32_t block_exclusive_max(uint32_t v, uint32_t carry, uint32_t* total,
                                                        uint32_t* smem) {
  constexpr unsigned kWaves = kThreads / 64;
  const unsigned lane = threadIdx.x & 63u, w = threadIdx.x / 64u;
  // inclusive running maximum over the wave with DPP moves (as wave_inclusive_sum; 0 is the identity), then the
  // lane before's value (wave_shr 1; lane 0 gets 0)
  uint32_t x = v;
  x = max(x, dpp_or_zero<0x111, 0xF>(x));
  x = max(x, dpp_or_zero<0x112, 0xF>(x));
  x = max(x, dpp_or_zero<0x114, 0xF>(x));
  x = max(x, dpp_or_zero<0x118, 0xF>(x));
  x = max(x, dpp_or_zero<0x142, 0xA>(x));
  x = max(x, dpp_or_zero<0x143, 0xC>(x));
  const uint32_t ex = dpp_or_zero<0x138, 0xF>(x);
  if (lane == 63) smem[w] = x;
  __syncthreads();
  uint32_t before = carry, all = carry;
#pragma unroll
  for (unsigned q = 0; q < kWaves; ++q) {
    const uint32_t m = smem[q];
    if (q < w) before = max(before, m);
    all = max(all, m);
  }
  __syncthreads();
  *total = all;
  return max(before, ex);
}

// Emission. Workgroup b owns emission positions [256 b, 256 b + 256) and the contiguous output range of their
// pairs, which it writes in chunks of 1024 pairs, four consecutive pairs per thread (coalesced stores; the chunks
// start at the range's first position rounded down to a multiple of four, so that each thread's four pairs are
// one aligned 16-byte vector of 32-bit keys or values, and the positions before the range are masked). In each
// chunk every splat marks the slot of its first pair with its position + 1, and a running maximum over the chunk
// (seeded with the previous chunk's last owner) gives each pair its splat. Inside a splat the tiles go row by
// row. 64-bit keys: (tile << 32) | depth bits; 32-bit keys: the tile id only, or with kPacked
// (tile << idx_bits) | splat and no value array.
template <typename K, bool kPacked = false>
__global__ __launch_bounds__(kThreads) void k_emit(const uint4* __restrict__ rects, const float* __restrict__ depths,
                                                   uint32_t n, const uint32_t* __restrict__ order,
                                                   uint32_t order_mask, uint32_t tiles_x,
                                                   const uint64_t* __restrict__ offsets, uint64_t pairs_cap,
                                                   const uint64_t* __restrict__ pairs_dev,
                                                   K* __restrict__ keys, uint32_t* __restrict__ vals,
                                                   uint32_t idx_bits) {
  constexpr uint32_t kPer = 4, kChunk = kPer * kThreads;  // kPer = 4: one 16-byte vector of values per thread
  __shared__ uint64_t s_off[kThreads + 1];
  __shared__ uint32_t s_tx0[kThreads], s_ty0[kThreads], s_w[kThreads], s_idx[kThreads], s_dbits[kThreads];
  __shared__ uint32_t s_mark[kChunk];
  __shared__ uint32_t smem[kThreads / kWave];
  const uint32_t tid = threadIdx.x;
  const uint32_t j = blockIdx.x * kThreads + tid;
  const uint64_t num_pairs = count_within(pairs_dev, pairs_cap);  // 0: nothing fits, nothing is written
  s_off[tid] = offsets[min(j, n)];
  if (tid == 0) s_off[kThreads] = offsets[min(blockIdx.x * kThreads + kThreads, n)];
  if (j < n) {
    uint32_t i = order ? order[j] & order_mask : j;
    if (i >= n) i = 0;  // not reachable with a permutation in `order`; its count is 0 then (see count_at)
    const uint4 r = rects[i];
    s_tx0[tid] = r.x;
    s_ty0[tid] = r.y;
    s_w[tid] = r.z ? r.z : 1u;
    s_idx[tid] = i;
    if constexpr (sizeof(K) == 8) s_dbits[tid] = __float_as_uint(depths[i]);
  }
  __syncthreads();
  const uint64_t begin = s_off[0], end = min(s_off[kThreads], num_pairs);
  const uint64_t my_start = s_off[tid];
  const bool has_pairs = s_off[tid + 1] > my_start;
  uint32_t carry = 0;
  for (uint64_t c0 = begin & ~uint64_t(kPer - 1); c0 < end; c0 += kChunk) {
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) s_mark[e * kThreads + tid] = 0;
    __syncthreads();
    // splats with pairs have distinct first positions
    if (has_pairs && my_start >= c0 && my_start < c0 + kChunk) s_mark[my_start - c0] = tid + 1;
    __syncthreads();
    uint32_t m[kPer];
    uint32_t run = 0;
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) {
      run = max(run, s_mark[kPer * tid + e]);
      m[e] = run;
    }
    uint32_t chunk_max;
    const uint32_t before = block_exclusive_max<kThreads>(run, carry, &chunk_max, smem);
    // the thread's kPer consecutive pairs; written as vectors when all of them are in the range (p0 is a multiple
    // of kPer, so the vectors are aligned: 16 bytes of 32-bit keys or values, 32 of 64-bit keys), element by
    // element at the ends of the range
    const uint64_t p0 = c0 + kPer * tid;
    K kk[kPer];
    uint32_t vv[kPer];
    bool ok[kPer];
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) {
      const uint64_t p = p0 + e;
      const uint32_t owner = max(before, m[e]);  // >= 1 for every pair below end
      ok[e] = p >= begin && p < end && owner > 0;
      const uint32_t q = owner > 0 ? owner - 1 : 0;
      const uint32_t k = uint32_t(p - s_off[q]);
      const uint32_t w = s_w[q];
      const uint32_t row = div_small(k, w);
      const uint64_t tile = uint64_t(s_ty0[q] + row) * tiles_x + (s_tx0[q] + (k - row * w));
      if constexpr (sizeof(K) == 8)
        kk[e] = (tile << 32) | s_dbits[q];
      else if constexpr (kPacked)
        kk[e] = K((uint32_t(tile) << idx_bits) | s_idx[q]);
      else
        kk[e] = K(tile);
      vv[e] = s_idx[q];
    }
    if (ok[0] && ok[1] && ok[2] && ok[3]) {
      if constexpr (sizeof(K) == 8) {
        reinterpret_cast<ulonglong2*>(keys + p0)[0] = make_ulonglong2(kk[0], kk[1]);
        reinterpret_cast<ulonglong2*>(keys + p0)[1] = make_ulonglong2(kk[2], kk[3]);
      } else {
        *reinterpret_cast<uint4*>(keys + p0) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
      }
      if constexpr (!kPacked) *reinterpret_cast<uint4*>(vals + p0) = make_uint4(vv[0], vv[1], vv[2], vv[3]);
    } else {
#pragma unroll
      for (uint32_t e = 0; e < kPer; ++e)
        if (ok[e]) {
          keys[p0 + e] = kk[e];
          if constexpr (!kPacked) vals[p0 + e] = vv[e];
        }
    }
    carry = chunk_max;
  }
}

// Emission under the ellipse rule: thread j walks its splat's box row by row and writes the kept tiles at
// offsets[j] onwards (each splat's pairs are contiguous; the stores are not coalesced across threads).
template <typename K, bool kPacked = false>
__global__ __launch_bounds__(kThreads) void k_emit_ellipse(const float* __restrict__ splats,
                                                           const uint4* __restrict__ rects,
                                                           const float* __restrict__ depths, uint32_t n,
                                                           const uint32_t* __restrict__ order, uint32_t order_mask,
                                                           uint32_t tiles_x,
                                                           const uint64_t* __restrict__ offsets,
                                                           uint64_t pairs_cap, const uint64_t* __restrict__ pairs_dev,
                                                           K* __restrict__ keys,
                                                           uint32_t* __restrict__ vals, uint32_t idx_bits) {
  const uint32_t j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= n) return;
  const uint32_t i = order ? order[j] & order_mask : j;
  if (i >= n) return;  // not reachable with a permutation in `order`
  const uint4 r = rects[i];
  const float* sp = splats + size_t(i) * 9;
  const float x = sp[0], y = sp[1], a = sp[2], b = sp[3], c = sp[4];
  const uint32_t dbits = __float_as_uint(depths[i]);
  uint64_t p = offsets[j];
  const uint64_t p_end = min(offsets[j + 1], count_within(pairs_dev, pairs_cap));
  // rect = (tx0, ty0, w, h)
  for (uint32_t ty = r.y; ty < r.y + r.w && p < p_end; ++ty)
    for (uint32_t tx = r.x; tx < r.x + r.z && p < p_end; ++tx) {
      if (!ellipse_meets_tile(x, y, a, b, c, tx, ty)) continue;
      const uint64_t tile = uint64_t(ty) * tiles_x + tx;
      if constexpr (sizeof(K) == 8)
        keys[p] = (tile << 32) | dbits;
      else if constexpr (kPacked)
        keys[p] = K((uint32_t(tile) << idx_bits) | i);
      else
        keys[p] = K(tile);
      if constexpr (!kPacked) vals[p] = i;
      ++p;
    }
}

// Fused counting sort of the pairs by tile (the tile-first scheme under the box rule), in place of emitting keys and
// radix-sorting them, and without the count scan; in two levels, tiles and super-tiles (squares of 2 x 2 tiles).
// Block b of kFuseBlock consecutive splats (in index order) computes their rectangles and counts, and counts its
// splats per tile and per super-tile with two difference arrays in LDS (four additions per splat and level: +1 at
// the rectangle's first corner, -1 past its right and bottom edges, +1 past both; prefix sums along x and then y
// turn them into the counts), written as row b of a [blocks][tiles + super-tiles] table (k_prep_rows). A column scan
// turns each row into the block's offset in each list and gives each list's total (k_tile_cols); scans of the
// totals give the tiles' starts with the ranges, and the super-tiles' starts (k_tile_starts). The same blocks then
// enumerate their (splat, super-tile) pairs - a third of the (splat, tile) pairs at 410k splats - and place each
// splat at the next free slot of their stretch of the super-tile's list (an LDS counter per super-tile;
// k_tile_scatter). Within a stretch the order is whatever the LDS atomics give: the per-super-tile order that
// follows (tile_depth.hip) sorts each list by (depth bits, splat), which is unique, and writes the four tiles'
// lists from it, so the bins do not depend on it. The pairs are enumerated as in k_emit (chunks of pairs, owner
// marks and a running maximum).
constexpr uint32_t kFuseThreads = 1024;                  // a splat per thread
constexpr uint32_t kFuseBlock = kFuseThreads;            // splats per block
constexpr uint32_t kFuseMaxTiles = 8192;                 // tiles (+ at most half as many super-tiles) counted in LDS
constexpr uint32_t kColTiles = 64, kColThreads = 1024;   // the column scan: 64 tiles by 16 stretches of rows
constexpr uint32_t kColParts = kColThreads / kColTiles;
constexpr uint32_t kColBatch = 32;                       // rows loaded at once
constexpr uint32_t kStartThreads = 1024, kStartPer = kFuseMaxTiles / kStartThreads;

// Logical block of physical block i of nb. Workgroups are dealt to the eight dies in turn (die i mod 8); this hands
// die x a contiguous run of logical blocks instead, so that each die writes one contiguous stretch of every tile's
// list and its L2 merges the partial lines of that stretch before they go to memory.
__device__ __forceinline__ uint32_t die_band(uint32_t i, uint32_t nb) {
  const uint32_t x = i % 8u, j = i / 8u, per = nb / 8u, rem = nb % 8u;
  return x * per + min(x, rem) + j;
}

// Enumerates the pairs of a block of kFuseBlock splats (thread tid holds splat tid of the block): s_off[0..kFuseBlock]
// are the splats' block-local first pair positions (s_off[kFuseBlock] = the block's total, `end` the pairs to
// enumerate, end <= that total), s_tx0 / s_ty0 / s_w their rectangles. Chunks of kPer pairs per thread, as k_emit.
// Calls f(q, row, col) for each pair, q the splat's index in the block and (col, row) the pair's cell of the grid.
// Every thread of the workgroup must call it.
template <typename F>
__device__ __forceinline__ void for_each_pair(const uint32_t* s_off, const uint32_t* s_tx0, const uint32_t* s_ty0,
                                              const uint32_t* s_w, uint32_t end, uint32_t* s_mark, uint32_t* smem,
                                              F f) {
  constexpr uint32_t kPer = 4, kChunk = kPer * kFuseThreads;
  const uint32_t tid = threadIdx.x;
  uint32_t carry = 0;
  for (uint32_t c0 = 0; c0 < end; c0 += kChunk) {
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) s_mark[e * kFuseThreads + tid] = 0;
    __syncthreads();
    {  // splats with pairs have distinct first positions
      const uint32_t first = s_off[tid];
      if (s_off[tid + 1] > first && first >= c0 && first < c0 + kChunk) s_mark[first - c0] = tid + 1;
    }
    __syncthreads();
    uint32_t m[kPer];
    uint32_t run = 0;
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) {
      run = max(run, s_mark[kPer * tid + e]);
      m[e] = run;
    }
    uint32_t chunk_max;
    const uint32_t before = block_exclusive_max<kFuseThreads>(run, carry, &chunk_max, smem);
    const uint32_t p0 = c0 + kPer * tid;
#pragma unroll
    for (uint32_t e = 0; e < kPer; ++e) {
      const uint32_t p = p0 + e;
      const uint32_t owner = max(before, m[e]);  // >= 1 for every pair below end
      if (p < end && owner > 0) {
        const uint32_t q = owner - 1;
        const uint32_t k = p - s_off[q];
        const uint32_t w = s_w[q];
        const uint32_t r = div_small(k, w);
        f(q, s_ty0[q] + r, s_tx0[q] + (k - r * w));
      }
    }
    carry = chunk_max;
  }
}

// Super-tiles of a grid of tiles_x x tiles_y tiles: ceil(tiles_x / 2) x ceil(tiles_y / 2), super-tile (sx, sy)
// holding tiles (2 sx + dx, 2 sy + dy), dx, dy in {0, 1}.
__host__ __device__ __forceinline__ uint32_t super_dim(uint32_t tiles) { return (tiles + 1) / 2; }

// Adds the rectangle [x0, x1) x [y0, y1) to the difference array d[ny][nx] in LDS (wrapping 32-bit sums): after
// inclusive prefix sums along x and then along y each of its cells holds one more. Corners past the last column or
// row are left out (nothing after them is summed).
__device__ __forceinline__ void diff_add(uint32_t* d, uint32_t nx, uint32_t ny, uint32_t x0, uint32_t y0,
                                         uint32_t x1, uint32_t y1) {
  atomicAdd(&d[y0 * nx + x0], 1u);
  if (x1 < nx) atomicAdd(&d[y0 * nx + x1], ~0u);
  if (y1 < ny) {
    atomicAdd(&d[y1 * nx + x0], ~0u);
    if (x1 < nx) atomicAdd(&d[y1 * nx + x1], 1u);
  }
}

// Inclusive prefix sums, in place in LDS, of `lines` sequences of `len` values: sequence k starts at a[k * step]
// and its values lie `stride` apart. The workgroup's waves take the sequences in turn, 64 values per step.
__device__ __forceinline__ void lds_scan_lines(uint32_t* a, uint32_t lines, uint32_t len, uint32_t step,
                                               uint32_t stride) {
  const uint32_t lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave, waves = blockDim.x / kWave;
  for (uint32_t k = w; k < lines; k += waves) {
    uint32_t* const line = a + k * step;
    uint32_t carry = 0;
    for (uint32_t c0 = 0; c0 < len; c0 += kWave) {
      const uint32_t i = c0 + lane;
      const uint32_t x = wave_inclusive_sum(i < len ? line[i * stride] : 0u) + carry;
      if (i < len) line[i * stride] = x;
      carry = uint32_t(__builtin_amdgcn_readlane(int(x), int(kWave - 1)));
    }
  }
}

// k_prep for the fused counting sort (box rule, num_tiles <= kFuseMaxTiles): blocks of kFuseBlock splats write
// each splat's rectangle and count, the block's count total in part[block] (k_total sums them), and the block's
// splats per tile and per super-tile as row `block` of `rows` ([blocks][tiles + super-tiles]).
__global__ __launch_bounds__(kFuseThreads) void k_prep_rows(const float* __restrict__ splats,
                                                            const float* __restrict__ depths, uint32_t n,
                                                            uint32_t tiles_x, uint32_t tiles_y,
                                                            uint4* __restrict__ rects, uint32_t* __restrict__ counts,
                                                            uint64_t* __restrict__ part,
                                                            uint32_t* __restrict__ rows) {
  extern __shared__ uint32_t s_cnt[];  // [tiles_y][tiles_x], then [sup_y][sup_x]: difference arrays, then counts
  __shared__ uint32_t smem[kFuseThreads / kWave];
  const uint32_t sup_x = super_dim(tiles_x), sup_y = super_dim(tiles_y);
  const uint32_t num_tiles = tiles_x * tiles_y, width = num_tiles + sup_x * sup_y;
  uint32_t* const s_sup = s_cnt + num_tiles;
  const uint32_t tid = threadIdx.x, i = blockIdx.x * kFuseBlock + tid;
  for (uint32_t t = tid; t < width; t += kFuseThreads) s_cnt[t] = 0;
  Rect r{0, 0, 0, 0};
  if (i < n) {
    r = tile_rect(splats + size_t(i) * 9, depths[i], tiles_x, tiles_y);
    rects[i] = make_uint4(r.tx0, r.ty0, r.w, r.h);
    counts[i] = r.w * r.h;
  }
  uint32_t total;  // the scan's barriers also order the zeroing before the additions
  block_exclusive_scan<uint32_t, kFuseThreads>(r.w * r.h, &total, smem);
  if (tid == 0) part[blockIdx.x] = total;
  if (r.w) {
    diff_add(s_cnt, tiles_x, tiles_y, r.tx0, r.ty0, r.tx0 + r.w, r.ty0 + r.h);
    diff_add(s_sup, sup_x, sup_y, r.tx0 / 2, r.ty0 / 2, (r.tx0 + r.w - 1) / 2 + 1, (r.ty0 + r.h - 1) / 2 + 1);
  }
  __syncthreads();
  lds_scan_lines(s_cnt, tiles_y, tiles_x, tiles_x, 1);  // along x
  lds_scan_lines(s_sup, sup_y, sup_x, sup_x, 1);
  __syncthreads();
  lds_scan_lines(s_cnt, tiles_x, tiles_y, 1, tiles_x);  // along y
  lds_scan_lines(s_sup, sup_x, sup_y, 1, sup_x);
  __syncthreads();
  uint32_t* const row = rows + size_t(blockIdx.x) * width;
  for (uint32_t t = tid; t < width; t += kFuseThreads) row[t] = s_cnt[t];
}

// The scatter: the workgroup takes block blk (die-banded) of kFuseBlock splats, enumerates its (splat, super-tile)
// pairs from the rectangles, and puts at list[sup_start[s] + rows[blk][num_tiles + s] + its slot] the pair's entry
// (depth bits << 32) | (cover << 28) | splat, cover the four bits (2 dy + dx) of the super-tile's tiles the splat's
// rectangle covers (rows and the starts as k_tile_cols and k_tile_starts leave them; n < 2^28). Nothing when the
// pairs exceed the capacity.
constexpr uint32_t kCoverShift = 28;
__global__ __launch_bounds__(kFuseThreads) void k_tile_scatter(const uint4* __restrict__ rects,
                                                               const float* __restrict__ depths, uint32_t n,
                                                               uint32_t tiles_x, uint32_t tiles_y, uint64_t pairs_cap,
                                                               const uint64_t* __restrict__ pairs_dev,
                                                               const uint32_t* __restrict__ rows,
                                                               const uint32_t* __restrict__ sup_start,
                                                               uint64_t* __restrict__ list) {
  extern __shared__ uint32_t s_tile[];  // a counter per super-tile
  __shared__ uint32_t s_off[kFuseBlock + 1], s_tx0[kFuseBlock], s_ty0[kFuseBlock], s_w[kFuseBlock];
  __shared__ uint32_t s_rx[kFuseBlock], s_ry[kFuseBlock], s_dbits[kFuseBlock];  // tile rectangle (x0 | w << 16, ..)
  __shared__ uint32_t s_mark[4 * kFuseThreads];
  __shared__ uint32_t smem[kFuseThreads / kWave];
  const uint32_t tid = threadIdx.x;
  const uint32_t sup_x = super_dim(tiles_x), num_tiles = tiles_x * tiles_y, num_sup = sup_x * super_dim(tiles_y);
  const uint32_t blk = die_band(blockIdx.x, gridDim.x);
  const uint32_t j0 = blk * kFuseBlock, i = j0 + tid;
  const uint32_t* const row = rows + size_t(blk) * (num_tiles + num_sup) + num_tiles;
  for (uint32_t t = tid; t < num_sup; t += kFuseThreads) s_tile[t] = sup_start[t] + row[t];
  uint32_t c = 0;
  uint32_t sx0 = 0, sy0 = 0, sw = 1;
  uint4 r = make_uint4(0, 0, 0, 0);
  if (i < n) {
    r = rects[i];
    if (r.z) {
      sx0 = r.x / 2, sy0 = r.y / 2;
      sw = (r.x + r.z - 1) / 2 - sx0 + 1;
      c = sw * ((r.y + r.w - 1) / 2 - sy0 + 1);
    }
  }
  s_tx0[tid] = sx0;
  s_ty0[tid] = sy0;
  s_w[tid] = sw;
  s_rx[tid] = r.x | (r.z << 16);  // tiles_x, tiles_y <= kFuseMaxTiles: 16 bits each
  s_ry[tid] = r.y | (r.w << 16);
  s_dbits[tid] = c ? __float_as_uint(depths[i]) : 0u;
  uint32_t total;
  s_off[tid] = block_exclusive_scan<uint32_t, kFuseThreads>(c, &total, smem);
  if (tid == 0) s_off[kFuseBlock] = total;
  const uint64_t cap = count_within(pairs_dev, pairs_cap);
  const uint32_t end = cap ? total : 0u;  // 0: nothing fits, nothing is written
  __syncthreads();
  for_each_pair(s_off, s_tx0, s_ty0, s_w, end, s_mark, smem, [&](uint32_t q, uint32_t sy, uint32_t sx) {
    const uint32_t rx = s_rx[q], ry = s_ry[q];
    uint32_t cover = 0;
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j)
      if (2 * sx + (j & 1u) - (rx & 0xFFFFu) < (rx >> 16) && 2 * sy + (j >> 1) - (ry & 0xFFFFu) < (ry >> 16))
        cover |= 1u << j;
    const uint32_t slot = atomicAdd(&s_tile[sy * sup_x + sx], 1u);
    if (slot < cap)  // always, when the counts agree; keeps a stray write in bounds
      list[slot] = (uint64_t(s_dbits[q]) << 32) | (cover << kCoverShift) | (j0 + q);
  });
}

// Column scan of the [nblk][num_tiles] count table (num_tiles: the row width, here tiles and super-tiles): each row
// becomes the block's exclusive offset within each list, and tile_total[column] receives the column's sum. A workgroup takes kColTiles tiles; its kColParts
// thread groups each sum a stretch of consecutive rows, then rewrite them starting from the sums of the stretches
// before. The row loads of 64 consecutive tiles are 256-byte segments.
__global__ __launch_bounds__(kColThreads) void k_tile_cols(uint32_t* __restrict__ rows, uint32_t nblk,
                                                           uint32_t num_tiles, uint32_t* __restrict__ tile_total) {
  __shared__ uint32_t s_sum[kColParts][kColTiles];
  const uint32_t lt = threadIdx.x % kColTiles, part = threadIdx.x / kColTiles;
  const uint32_t t = blockIdx.x * kColTiles + lt;
  const uint32_t per = (nblk + kColParts - 1) / kColParts;
  const uint32_t b0 = min(nblk, part * per), b1 = min(nblk, b0 + per);
  const bool live = t < num_tiles;
  uint32_t sum = 0;
  for (uint32_t c = b0; c < b1; c += kColBatch) {
    uint32_t v[kColBatch];
#pragma unroll
    for (uint32_t i = 0; i < kColBatch; ++i) v[i] = live && c + i < b1 ? rows[size_t(c + i) * num_tiles + t] : 0u;
#pragma unroll
    for (uint32_t i = 0; i < kColBatch; ++i) sum += v[i];
  }
  s_sum[part][lt] = sum;
  __syncthreads();
  uint32_t run = 0, total = 0;
#pragma unroll
  for (uint32_t q = 0; q < kColParts; ++q) {
    const uint32_t x = s_sum[q][lt];
    if (q < part) run += x;
    total += x;
  }
  if (!live) return;
  if (part == 0) tile_total[t] = total;
  for (uint32_t c = b0; c < b1; c += kColBatch) {
    uint32_t v[kColBatch];
#pragma unroll
    for (uint32_t i = 0; i < kColBatch; ++i) v[i] = c + i < b1 ? rows[size_t(c + i) * num_tiles + t] : 0u;
#pragma unroll
    for (uint32_t i = 0; i < kColBatch; ++i) {
      if (c + i < b1) rows[size_t(c + i) * num_tiles + t] = run;
      run += v[i];
    }
  }
}

// One workgroup: start[0..num_tiles) = the exclusive scan of total[0..num_tiles) with the ranges [start, start +
// total), and start[num_tiles..+num_sup) = the exclusive scan of the super-tiles' totals (each at most kFuseMaxTiles
// entries, kStartPer consecutive ones per thread); every range empty when the pairs exceed the capacity.
__global__ __launch_bounds__(kStartThreads) void k_tile_starts(const uint32_t* __restrict__ total, uint32_t num_tiles,
                                                               uint32_t num_sup, uint64_t pairs_cap,
                                                               const uint64_t* __restrict__ pairs_dev,
                                                               uint32_t* __restrict__ start,
                                                               uint32_t* __restrict__ ranges) {
  __shared__ uint32_t smem[kStartThreads / kWave];
  const bool fits = count_within(pairs_dev, pairs_cap) > 0;
  for (uint32_t level = 0; level < 2; ++level) {
    const uint32_t off = level ? num_tiles : 0u, count = level ? num_sup : num_tiles;
    const uint32_t t0 = threadIdx.x * kStartPer;
    uint32_t v[kStartPer], sum = 0;
#pragma unroll
    for (uint32_t i = 0; i < kStartPer; ++i) {
      v[i] = fits && t0 + i < count ? total[off + t0 + i] : 0u;
      sum += v[i];
    }
    uint32_t run = block_exclusive_scan<uint32_t, kStartThreads>(sum, nullptr, smem);
#pragma unroll
    for (uint32_t i = 0; i < kStartPer; ++i)
      if (t0 + i < count) {
        start[off + t0 + i] = run;
        if (!level) {
          ranges[2 * (t0 + i)] = run;
          ranges[2 * (t0 + i) + 1] = run + v[i];
        }
        run += v[i];
      }
  }
}

// Per-tile ranges from the sorted keys: the boundary between pairs i-1 and i (i in [0, P]) opens the ranges of
// the tiles after the previous pair's and closes those before the current pair's. Each thread takes kRangeItems
// consecutive boundaries (16-byte loads of 32-bit keys). With keys_final (the presort scheme when no sort pass
// ran) it also writes the final 64-bit keys (tile << 32 | depth bits). 32-bit keys hold the tile id above bit
// tile_shift (packed keys; 0 otherwise).
constexpr uint32_t kRangeItems = 4;

template <typename K>
__global__ __launch_bounds__(kThreads) void k_ranges(const K* __restrict__ keys, const uint32_t* __restrict__ vals,
                                                     uint64_t pairs_cap, const uint64_t* __restrict__ pairs_dev,
                                                     uint32_t num_tiles,
                                                     const float* __restrict__ depths, uint32_t n,
                                                     uint64_t* __restrict__ keys_final,
                                                     uint32_t* __restrict__ ranges, uint32_t tile_shift) {
  const uint64_t P = count_within(pairs_dev, pairs_cap);  // 0 when nothing fitted: every range is then empty
  const uint64_t i0 = (uint64_t(blockIdx.x) * kThreads + threadIdx.x) * kRangeItems;
  if (i0 > P) return;
  auto tile_of = [tile_shift](K k) -> int64_t {
    return sizeof(K) == 8 ? int64_t(uint64_t(k) >> 32) : int64_t(uint32_t(k) >> tile_shift);
  };
  // tiles of pairs i0 - 1 .. i0 + kRangeItems - 1 (-1 before the first pair, num_tiles from pair P on)
  int64_t t[kRangeItems + 1];
  uint32_t v[kRangeItems];
  t[0] = i0 == 0 ? -1 : tile_of(keys[i0 - 1]);
  if (sizeof(K) == 4 && i0 + kRangeItems <= P) {
    const uint4 kk = *reinterpret_cast<const uint4*>(keys + i0);
    t[1] = kk.x >> tile_shift, t[2] = kk.y >> tile_shift, t[3] = kk.z >> tile_shift, t[4] = kk.w >> tile_shift;
  } else {
#pragma unroll
    for (uint32_t q = 0; q < kRangeItems; ++q) t[q + 1] = i0 + q < P ? tile_of(keys[i0 + q]) : int64_t(num_tiles);
  }
  if (keys_final) {
    if (i0 + kRangeItems <= P) {
      const uint4 vv = *reinterpret_cast<const uint4*>(vals + i0);
      v[0] = vv.x, v[1] = vv.y, v[2] = vv.z, v[3] = vv.w;
    } else {
#pragma unroll
      for (uint32_t q = 0; q < kRangeItems; ++q) v[q] = i0 + q < P ? vals[i0 + q] : 0u;
    }
  }
#pragma unroll
  for (uint32_t q = 0; q < kRangeItems; ++q) {
    const uint64_t i = i0 + q;
    const int64_t prev = t[q], cur = t[q + 1];
    if (i <= P && cur != prev) {
      for (int64_t u = prev + 1; u <= cur && u < int64_t(num_tiles); ++u) ranges[2 * u] = uint32_t(i);
      for (int64_t u = prev < 0 ? 0 : prev; u < cur && u < int64_t(num_tiles); ++u) ranges[2 * u + 1] = uint32_t(i);
    }
  }
  if (keys_final) {
    uint64_t f[kRangeItems];
#pragma unroll
    for (uint32_t q = 0; q < kRangeItems; ++q)
      f[q] = (uint64_t(t[q + 1]) << 32) | (v[q] < n ? __float_as_uint(depths[v[q]]) : 0u);
    if (i0 + kRangeItems <= P) {
      ulonglong2* dst = reinterpret_cast<ulonglong2*>(keys_final + i0);
      dst[0] = make_ulonglong2(f[0], f[1]);
      dst[1] = make_ulonglong2(f[2], f[3]);
    } else {
#pragma unroll
      for (uint32_t q = 0; q < kRangeItems; ++q)
        if (i0 + q < P) keys_final[i0 + q] = f[q];
    }
  }
}

// Longest lists first, so that the raster kernels start the slowest tiles at once and the short ones fill the
// workgroup slots that free up (the tile loads differ several-fold, and the grid exceeds the resident slots). A
// counting sort of the tiles into 64 classes of list length (or of the previous forward's walk counts): most tiles
// fall into a few classes, so each wave first groups its lanes by class (a ballot per class bit) and one lane per
// class does the LDS addition for all of them. Each thread keeps the lengths of its first kOrderItems tiles in
// registers; further tiles are read again in each pass.
constexpr uint32_t kOrderThreads = 1024, kOrderClasses = 64, kOrderItems = 4;
static_assert(kOrderClasses == kWave, "one class per lane in the scan");

__global__ __launch_bounds__(kOrderThreads) void k_tile_order(const uint32_t* __restrict__ ranges,
                                                              const uint32_t* __restrict__ cost, uint32_t num_tiles,
                                                              uint32_t num_pairs, uint32_t* __restrict__ order,
                                                              bool identity) {
  __shared__ uint32_t s_count[kOrderClasses], s_base[kOrderClasses];
  __shared__ uint32_t s_max[kOrderThreads / kWave];
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  if (identity) {
    for (uint32_t t = tid; t < num_tiles; t += kOrderThreads) order[t] = t;
    return;
  }
  auto len_of = [&](uint32_t t) -> uint32_t {
    if (cost) {
      const uint4 c = reinterpret_cast<const uint4*>(cost)[t];
      return c.x + c.y + c.z + c.w;
    }
    const uint32_t start = min(ranges[2 * t], num_pairs);
    const uint32_t end = max(start, min(ranges[2 * t + 1], num_pairs));
    return end - start;
  };
  if (tid < kOrderClasses) s_count[tid] = 0;
  uint32_t len[kOrderItems];
  uint32_t lmax = 0;
#pragma unroll
  for (uint32_t i = 0; i < kOrderItems; ++i) {
    const uint32_t t = tid + i * kOrderThreads;
    len[i] = t < num_tiles ? len_of(t) : 0u;
    lmax = max(lmax, len[i]);
  }
  for (uint32_t t = tid + kOrderItems * kOrderThreads; t < num_tiles; t += kOrderThreads) lmax = max(lmax, len_of(t));
  for (uint32_t d = 1; d < kWave; d <<= 1) lmax = max(lmax, uint32_t(__shfl_xor(int(lmax), int(d))));
  if (lane == 0) s_max[w] = lmax;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (uint32_t q = 0; q < kOrderThreads / kWave; ++q) m = max(m, s_max[q]);
  const uint64_t span = uint64_t(m) + 1;
  auto class_of = [&](uint32_t l) {  // 0 = longest
    return kOrderClasses - 1 - uint32_t(uint64_t(l) * kOrderClasses / span);
  };
  // f(t, valid, class) for every tile, in chunks of kOrderThreads that every thread of the workgroup takes part in
  auto for_each_tile = [&](auto f) {
#pragma unroll
    for (uint32_t i = 0; i < kOrderItems; ++i) {
      if (i * kOrderThreads >= num_tiles) return;
      const uint32_t t = tid + i * kOrderThreads;
      f(t, t < num_tiles, class_of(len[i]));
    }
    for (uint32_t t0 = kOrderItems * kOrderThreads; t0 < num_tiles; t0 += kOrderThreads) {
      const uint32_t t = t0 + tid;
      f(t, t < num_tiles, class_of(t < num_tiles ? len_of(t) : 0u));
    }
  };
  for_each_tile([&](uint32_t, bool valid, uint32_t c) {
    const uint64_t peers = match_digit<6>(c, valid);
    if (valid && (peers & lanemask_lt(lane)) == 0) atomicAdd(&s_count[c], uint32_t(__popcll(peers)));
  });
  __syncthreads();
  if (w == 0) {
    const uint32_t x = s_count[lane];
    s_base[lane] = wave_inclusive_sum(x) - x;
  }
  __syncthreads();
  for_each_tile([&](uint32_t t, bool valid, uint32_t c) {
    const uint64_t peers = match_digit<6>(c, valid);
    const int leader = valid ? int(__ffsll(static_cast<unsigned long long>(peers))) - 1 : 0;
    uint32_t base = 0;
    if (valid && int(lane) == leader) base = atomicAdd(&s_base[c], uint32_t(__popcll(peers)));
    base = uint32_t(__shfl(int(base), leader));
    if (valid) order[base + uint32_t(__popcll(peers & lanemask_lt(lane)))] = t;
  });
}

uint32_t bits_of(uint64_t v) {
  uint32_t b = 0;
  for (; v; v >>= 1) ++b;
  return b;
}

uint32_t grid_for(uint64_t items, uint32_t per_block) { return uint32_t((items + per_block - 1) / per_block); }

}  // namespace
}  // namespace gsr

namespace gsr {

void launch_tile_order(hipStream_t s, const uint32_t* ranges, const uint32_t* cost, uint32_t num_tiles,
                       uint32_t num_pairs, uint32_t* order, bool identity) {
  if (num_tiles)
    hipLaunchKernelGGL(k_tile_order, dim3(1), dim3(kOrderThreads), 0, s, ranges, cost, num_tiles, num_pairs, order,
                       identity);
}

const uint32_t* raster_tile_order(gsr_ctx* ctx, hipStream_t s, const gsr_bins* bins, bool backward,
                                  gsr_status* st) {
  Arena& a = ctx->arena;
  const uint64_t num_tiles = uint64_t(bins->tiles_x) * bins->tiles_y;
  *st = GSR_OK;
  if (backward && ctx->order_ranges == bins->ranges && ctx->order_tiles == num_tiles && a.tile_order_ext.ptr)
    return static_cast<const uint32_t*>(a.tile_order_ext.ptr);
  if ((*st = grow(ctx, a.tile_order_ext, size_t(num_tiles) * 4))) return nullptr;
  uint32_t* order = static_cast<uint32_t*>(a.tile_order_ext.ptr);
  const uint32_t* cost = ctx->tile_order == GSR_ORDER_COST && ctx->cost_tiles == num_tiles
                             ? static_cast<const uint32_t*>(a.tile_cost.ptr) : nullptr;
  launch_tile_order(s, bins->ranges, cost, uint32_t(num_tiles), bins->num_pairs, order,
                    ctx->tile_order == GSR_ORDER_NONE);
  ctx->order_ranges = backward ? nullptr : bins->ranges;
  ctx->order_tiles = num_tiles;
  return order;
}

}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_bin(gsr_ctx* ctx, void* stream, const float* splats, const float* depths, uint32_t n,
                              uint32_t width, uint32_t height, gsr_bins* out) {
  if (!ctx || !out) return GSR_EINVAL;
  if (width == 0 || height == 0) return fail(ctx, GSR_EINVAL, "gsr_bin: empty image %ux%u", width, height);
  if (n && (!splats || !depths)) return fail(ctx, GSR_EINVAL, "gsr_bin: null splats or depths");
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  const uint64_t num_tiles = uint64_t(tiles_x) * tiles_y;
  if (num_tiles >= (uint64_t(1) << 32)) return fail(ctx, GSR_EINVAL, "gsr_bin: too many tiles");
  gsr_status st = enter(ctx);
  if (st) return st;
  ctx->order_ranges = nullptr;  // the ranges are rewritten: rank again before the next raster launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  Arena& a = ctx->arena;
  const bool ellipse = ctx->bin_rule == GSR_BIN_ELLIPSE;
  // An earlier call's pair count that has arrived in the meantime raises the capacity hint (before this call's
  // launch overwrites the pinned word).
  if (ctx->pairs_pending && hipEventQuery(a.total_ready) == hipSuccess) note_pair_count(ctx);
  // The tile-first scheme's two-level counting sort (box rule, the per-tile and per-super-tile counters fit LDS,
  // splat indices below the cover bits) orders long lists in chunks on chip. Its other form sorts each tile's list
  // on chip and longer ones through the arena; there, when the last count seen puts the average list beyond
  // kTileFirstAvg pairs, the presort scheme takes the call instead. All give the same bins bit for bit; the choice
  // is only about speed.
  const bool fusable = !ellipse && n && n < (1u << kCoverShift) && num_tiles <= kFuseMaxTiles;
  const bool tile_first = ctx->bin_scheme == GSR_BIN_TILE_DEPTH &&
                          (fusable || ctx->last_pairs <= uint64_t(kTileFirstAvg) * num_tiles);
  const bool presort = ctx->bin_scheme == GSR_BIN_PRESORT || (ctx->bin_scheme == GSR_BIN_TILE_DEPTH && !tile_first);
  const bool fused = tile_first && fusable;
  // Without a wait only once there is a count or a reservation to size the pair buffers from.
  const bool sync_free = ctx->bin_sync_free && n && (ctx->pair_hint > 0 || ctx->pair_reserved > 0);

  if ((st = grow(ctx, a.ranges, size_t(num_tiles) * 8))) return st;
  if ((st = grow(ctx, a.counts, size_t(n + 1) * 4)) || (st = grow(ctx, a.offsets, size_t(n + 1) * 8)) ||
      (st = grow(ctx, a.rects, size_t(n + 1) * 16)))
    return st;
  const uint32_t nb_prep = grid_for(n, kThreads), nb_scan = grid_for(n, kScanBlock);
  if ((st = grow(ctx, a.scan_part, size_t(std::max(nb_prep, nb_scan) + 1) * 8))) return st;
  if (presort && n) {
    if ((st = grow(ctx, a.order, size_t(n) * 8)) || (st = grow(ctx, a.order_alt, size_t(n) * 8)) ||
        (st = grow(ctx, a.order_vals, size_t(n) * 4)) || (st = grow(ctx, a.order_vals_alt, size_t(n) * 4)))
      return st;
  }
  uint4* rects = static_cast<uint4*>(a.rects.ptr);
  uint32_t* counts = static_cast<uint32_t*>(a.counts.ptr);
  uint64_t* offsets = static_cast<uint64_t*>(a.offsets.ptr);
  uint64_t* part = static_cast<uint64_t*>(a.scan_part.ptr);
  uint32_t* ok = static_cast<uint32_t*>(a.order.ptr);
  uint32_t* ov = static_cast<uint32_t*>(a.order_vals.ptr);
  // the presort scheme carries each splat's count in its depth-sort value when index and count fit 32 bits
  // (a count is at most num_tiles)
  const uint32_t idx_bits = bits_of(n ? n - 1 : 0);
  const bool pack_counts = presort && n && idx_bits + bits_of(num_tiles) <= 32;
  const uint32_t count_shift = pack_counts ? idx_bits : 32u;
  const uint32_t order_mask = pack_counts ? (idx_bits ? (1u << idx_bits) - 1u : 0u) : ~0u;

  // Rectangles, counts and the pair total first; the total goes to the host (a pinned word k_total writes) while
  // the depth sort runs.
  timing_mark(ctx, GSR_STAGE_BIN, s, false);
  hipError_t e = hipSuccess;
  // Sync-free, the launches are sized for a capacity: the capacity rule of the C0 resident arena page (section 2
  // table, row "C0"), the largest of 2^16 pairs, 16 per splat and 1.5 times the count seen, here also of a
  // reservation.
  const uint64_t capacity =
      sync_free ? std::min<uint64_t>(std::max<uint64_t>({ctx->pair_reserved, uint64_t(1) << 16, uint64_t(n) * 16,
                                                         ctx->pair_hint + ctx->pair_hint / 2}),
                                     (uint64_t(1) << 32) - 1)
                : 0;
  const uint32_t nb_fuse = grid_for(n, kFuseBlock);
  // the fused counting sort's lists: the tiles, then the super-tiles (2 x 2 tiles)
  const uint32_t num_sup = super_dim(tiles_x) * super_dim(tiles_y);
  const uint32_t lists = uint32_t(num_tiles) + num_sup;
  uint32_t* rows = nullptr;
  uint32_t* list_total = nullptr;
  uint32_t* list_start = nullptr;
  if (fused) {
    // the counting sort's count table, its column scan and the list starts (with the tile ranges) need no pair
    // count: they are queued before the wait for it
    if ((st = grow(ctx, a.tile_rows, (size_t(nb_fuse) + 2) * lists * 4))) return st;
    rows = static_cast<uint32_t*>(a.tile_rows.ptr);
    list_total = rows + size_t(nb_fuse) * lists;
    list_start = list_total + lists;
    hipLaunchKernelGGL(k_prep_rows, dim3(nb_fuse), dim3(kFuseThreads), size_t(lists) * 4, s, splats, depths, n,
                       tiles_x, tiles_y, rects, counts, part, rows);
    hipLaunchKernelGGL(k_total, dim3(1), dim3(kThreads), 0, s, static_cast<const uint64_t*>(part), nb_fuse,
                       offsets + n, a.host_total_dev);
    e = hipEventRecord(a.total_ready, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bin pair count readback");
    timing_mark(ctx, GSR_STAGE_TILE_SCAN, s, false);
    hipLaunchKernelGGL(k_tile_cols, dim3(grid_for(lists, kColTiles)), dim3(kColThreads), 0, s, rows, nb_fuse, lists,
                       list_total);
    hipLaunchKernelGGL(k_tile_starts, dim3(1), dim3(kStartThreads), 0, s, static_cast<const uint32_t*>(list_total),
                       uint32_t(num_tiles), num_sup, sync_free ? capacity : ~uint64_t(0),
                       sync_free ? static_cast<const uint64_t*>(offsets + n) : static_cast<const uint64_t*>(nullptr),
                       list_start, static_cast<uint32_t*>(a.ranges.ptr));
    timing_mark(ctx, GSR_STAGE_TILE_SCAN, s, true);
  } else if (n) {
    hipLaunchKernelGGL(k_prep, dim3(nb_prep), dim3(kThreads), 0, s, splats, depths, n, tiles_x, tiles_y, ellipse,
                       rects, counts,
                       presort ? ok : static_cast<uint32_t*>(nullptr), presort ? ov : static_cast<uint32_t*>(nullptr),
                       count_shift, part);
    hipLaunchKernelGGL(k_total, dim3(1), dim3(kThreads), 0, s, static_cast<const uint64_t*>(part), nb_prep,
                       offsets + n, a.host_total_dev);
  }
  if (n) {
    if ((st = check_launch(ctx, "gsr_bin rectangles"))) return st;
    if (!fused) e = hipEventRecord(a.total_ready, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bin pair count readback");
    ctx->pairs_pending = true;  // this call's count, on its way to the pinned word
    ctx->last_cap = 0;
  } else {
    ctx->pairs_pending = false;
    ctx->last_pairs = 0;
    ctx->last_cap = 0;
  }

  const uint32_t* order = nullptr;
  if (presort && n) {
    // 4 passes (even): the sorted result lands back in (order, order_vals)
    timing_mark(ctx, GSR_STAGE_DEPTH_SORT, s, false);
    st = radix_sort_launch<uint32_t>(ctx, s, ok, ov, n, 32, ok, ov, static_cast<uint32_t*>(a.order_alt.ptr),
                                     static_cast<uint32_t*>(a.order_vals_alt.ptr));
    if (st) return st;
    timing_mark(ctx, GSR_STAGE_DEPTH_SORT, s, true);
    order = ov;
  }
  // offsets in emission order (depth order for the presort scheme); the scan rewrites offsets[n] with the same total.
  // The fused counting sort enumerates each block's pairs from a block scan of its counts instead.
  if (n && !fused) {
    if (pack_counts) {
      // the sorted values carry the counts: both launches read them in place
      hipLaunchKernelGGL(k_scan_reduce, dim3(nb_scan), dim3(kThreads), 0, s, static_cast<const uint32_t*>(ov),
                         static_cast<const uint32_t*>(nullptr), count_shift, n, part, static_cast<uint32_t*>(nullptr),
                         a.done, a.done, offsets);
      hipLaunchKernelGGL(k_scan_down, dim3(nb_scan), dim3(kThreads), 0, s, static_cast<const uint32_t*>(ov),
                         static_cast<const uint32_t*>(nullptr), count_shift, n, part, offsets);
    } else {
      // otherwise the presort scheme gathers its counts once, into the depth sort's (now free) value scratch
      uint32_t* ordered = order ? static_cast<uint32_t*>(a.order_vals_alt.ptr) : nullptr;
      hipLaunchKernelGGL(k_scan_reduce, dim3(nb_scan), dim3(kThreads), 0, s, counts, order, 0u, n, part, ordered,
                         a.done, a.done, offsets);
      hipLaunchKernelGGL(k_scan_down, dim3(nb_scan), dim3(kThreads), 0, s, order ? ordered : counts,
                         static_cast<const uint32_t*>(nullptr), 0u, n, part, offsets);
    }
  }
  if ((st = check_launch(ctx, "gsr_bin depth sort/scan"))) return st;

  // The one wait of the call: the pair count sizes the arena and the launches below. Sync-free, the launches are
  // sized for a capacity instead and read the count from device memory (offsets[n], the scan's total); when it
  // exceeds the capacity they emit nothing and every tile's range is empty (gsr_bin_pair_count reports it).
  uint64_t P = 0;  // the pair count, or the capacity the launches are sized for
  const uint64_t* pairs_dev = nullptr;
  if (sync_free) {
    P = capacity;
    pairs_dev = offsets + n;
    ctx->last_cap = P;
  } else if (n) {
    e = hipEventSynchronize(a.total_ready);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bin pair count readback");
    note_pair_count(ctx);
    P = ctx->last_pairs;
    ctx->last_cap = P;
  }
  if (P >= (uint64_t(1) << 32)) return fail(ctx, GSR_EOVERFLOW, "gsr_bin: %llu pairs exceed 2^32 - 1",
                                            (unsigned long long)P);

  for (int q = 0; q < 2; ++q)
    if ((st = grow(ctx, a.keys[q], size_t(P) * 8)) || (st = grow(ctx, a.vals[q], size_t(P) * 4))) return st;
  if (tile_first && !fused && (st = grow(ctx, a.tile_scratch, size_t(P) * 8))) return st;
  uint32_t* v0 = static_cast<uint32_t*>(a.vals[0].ptr);
  uint32_t* ranges = static_cast<uint32_t*>(a.ranges.ptr);
  const uint32_t tile_bits = bits_of(num_tiles - 1);
  int res = 0;
  uint64_t* final_k = nullptr;
  uint32_t* sorted_v = nullptr;
  // the splat index and the tile id share one 32-bit key when they fit (and there is a tile pass to unpack it)
  const bool packed = presort && n && P > 0 && tile_bits > 0 && idx_bits + tile_bits <= 32;
  if (packed) {
    uint32_t* kb[2] = {static_cast<uint32_t*>(a.keys[0].ptr), static_cast<uint32_t*>(a.keys[1].ptr)};
    if (ellipse)
      hipLaunchKernelGGL((k_emit_ellipse<uint32_t, true>), dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, splats,
                         rects, depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0],
                         static_cast<uint32_t*>(nullptr), idx_bits);
    else
      hipLaunchKernelGGL((k_emit<uint32_t, true>), dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, rects, depths,
                         n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0], static_cast<uint32_t*>(nullptr),
                         idx_bits);
    res = (sort_passes(tile_bits) & 1u) ? 1 : 0;  // the first pass writes buffer 1 either way
    if (ctx->bin_keys) {
      if ((st = grow(ctx, a.order_alt, std::max<size_t>(size_t(n) * 8, size_t(P) * 8)))) return st;
      final_k = static_cast<uint64_t*>(a.order_alt.ptr);
    }
    timing_mark(ctx, GSR_STAGE_TILE_SORT, s, false);
    st = radix_sort_tiles_packed(ctx, s, kb[0], P, idx_bits, tile_bits, kb[res], kb[1 - res], v0, final_k,
                                 depths, n, pairs_dev);
    if (st) return st;
    timing_mark(ctx, GSR_STAGE_TILE_SORT, s, true);
    hipLaunchKernelGGL(k_ranges<uint32_t>, dim3(grid_for(P + 1, kThreads * kRangeItems)), dim3(kThreads), 0, s,
                       kb[res], static_cast<const uint32_t*>(v0), P, pairs_dev, uint32_t(num_tiles), depths, n,
                       static_cast<uint64_t*>(nullptr), ranges, idx_bits);
    sorted_v = v0;
  } else if (fused) {
    // the counting sort's scatter into the super-tiles' lists (the count table and the starts are queued above; a
    // super-tile's list is no longer than its tiles' lists together, so P entries hold them), then each super-tile
    // sorts its list by (depth, splat) on chip and writes its tiles' lists (tile_depth.hip); the lists' 64-bit
    // entries go in the scratch the other tile-first path uses for long lists
    if ((st = grow(ctx, a.tile_scratch, size_t(P) * 8))) return st;
    uint64_t* list = static_cast<uint64_t*>(a.tile_scratch.ptr);
    timing_mark(ctx, GSR_STAGE_TILE_SORT, s, false);
    hipLaunchKernelGGL(k_tile_scatter, dim3(nb_fuse), dim3(kFuseThreads), size_t(num_sup) * 4, s,
                       static_cast<const uint4*>(rects), depths, n, tiles_x, tiles_y, P, pairs_dev,
                       static_cast<const uint32_t*>(rows), static_cast<const uint32_t*>(list_start + num_tiles),
                       list);
    timing_mark(ctx, GSR_STAGE_TILE_SORT, s, true);
    if (ctx->bin_keys) {
      if ((st = grow(ctx, a.order_alt, std::max<size_t>(size_t(n) * 8, size_t(P) * 8)))) return st;
      final_k = static_cast<uint64_t*>(a.order_alt.ptr);
    }
    uint32_t* k0 = static_cast<uint32_t*>(a.keys[0].ptr);
    uint32_t* k1 = static_cast<uint32_t*>(a.keys[1].ptr);
    timing_mark(ctx, GSR_STAGE_TILE_DEPTH, s, false);
    launch_super_order(s, list, list_start + num_tiles, list_total + num_tiles, num_sup, tiles_x, tiles_y, ranges, P,
                       pairs_dev, depths, n, v0, final_k, k0, k0 + P, k1, k1 + P);
    timing_mark(ctx, GSR_STAGE_TILE_DEPTH, s, true);
    sorted_v = v0;
  } else if (tile_first) {
    // Pairs emitted splat by splat (index order), sorted stably by tile alone, then each tile's list by depth on
    // chip (tile_depth.hip): splat and tile id packed in one word when they fit, else tile ids with a splat array.
    uint32_t* kb[2] = {static_cast<uint32_t*>(a.keys[0].ptr), static_cast<uint32_t*>(a.keys[1].ptr)};
    const bool tpacked = tile_bits > 0 && idx_bits + tile_bits <= 32;
    if ((st = grow(ctx, a.order_vals_alt, std::max<size_t>(size_t(n) * 4, size_t(P) * 4)))) return st;
    uint32_t* spare = static_cast<uint32_t*>(a.order_vals_alt.ptr);  // a pair-count array for long tiles
    if (n) {
      if (tpacked) {
        if (ellipse)
          hipLaunchKernelGGL((k_emit_ellipse<uint32_t, true>), dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s,
                             splats, rects, depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0],
                             static_cast<uint32_t*>(nullptr), idx_bits);
        else
          hipLaunchKernelGGL((k_emit<uint32_t, true>), dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, rects,
                             depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0],
                             static_cast<uint32_t*>(nullptr), idx_bits);
      } else {
        if (ellipse)
          hipLaunchKernelGGL(k_emit_ellipse<uint32_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, splats,
                             rects, depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
        else
          hipLaunchKernelGGL(k_emit<uint32_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, rects, depths, n,
                             order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
      }
    }
    // the tile-sorted list (list, and list_vals when unpacked), where the result goes, and four pair-count arrays
    // free for lists longer than the on-chip capacity: the key buffers are 8 bytes per pair, so a list of 32-bit
    // words leaves the second half of its buffer free
    const uint32_t* list = kb[0];
    const uint32_t* list_vals = tpacked ? nullptr : v0;
    uint32_t* vals_out = tpacked ? v0 : static_cast<uint32_t*>(a.vals[1].ptr);
    uint32_t* scratch[4] = {kb[1], kb[1] + P, kb[0] + P, tpacked ? static_cast<uint32_t*>(a.vals[1].ptr) : spare};
    if (tile_bits > 0 && P > 0) {
      res = (sort_passes(tile_bits) & 1u) ? 1 : 0;
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, false);
      if (tpacked) {
        st = radix_sort_tiles_packed(ctx, s, kb[0], P, idx_bits, tile_bits, kb[res], kb[1 - res],
                                     static_cast<uint32_t*>(nullptr), static_cast<uint64_t*>(nullptr),
                                     static_cast<const float*>(nullptr), 0u, pairs_dev);
      } else {
        uint32_t* vr = static_cast<uint32_t*>(a.vals[res].ptr);
        uint32_t* vt = static_cast<uint32_t*>(a.vals[1 - res].ptr);
        st = radix_sort_launch<uint32_t>(ctx, s, kb[0], v0, P, tile_bits, kb[res], vr, kb[1 - res], vt, pairs_dev);
        list_vals = vr;
        vals_out = vt;
      }
      if (st) return st;
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, true);
      list = kb[res];
      scratch[0] = kb[1 - res];
      scratch[1] = kb[1 - res] + P;
      scratch[2] = kb[res] + P;
    }
    hipLaunchKernelGGL(k_ranges<uint32_t>, dim3(grid_for(P + 1, kThreads * kRangeItems)), dim3(kThreads), 0, s,
                       list, list_vals, P, pairs_dev, uint32_t(num_tiles), depths, n,
                       static_cast<uint64_t*>(nullptr), ranges, tpacked ? idx_bits : 0u);
    if (ctx->bin_keys) {
      if ((st = grow(ctx, a.order_alt, std::max<size_t>(size_t(n) * 8, size_t(P) * 8)))) return st;
      final_k = static_cast<uint64_t*>(a.order_alt.ptr);
    }
    timing_mark(ctx, GSR_STAGE_TILE_DEPTH, s, false);
    launch_tile_depth(s, list, list_vals, tpacked ? idx_bits : 32u, true, ranges, P, pairs_dev, uint32_t(num_tiles),
                      depths, n, vals_out, final_k, static_cast<uint64_t*>(a.tile_scratch.ptr), scratch[0],
                      scratch[1], scratch[2], scratch[3]);
    timing_mark(ctx, GSR_STAGE_TILE_DEPTH, s, true);
    sorted_v = vals_out;
  } else if (presort) {
    // tile ids as 32-bit keys, sorted by their tile_bits low bits
    uint32_t* kb[2] = {static_cast<uint32_t*>(a.keys[0].ptr), static_cast<uint32_t*>(a.keys[1].ptr)};
    if (n)
    {
      if (ellipse)
        hipLaunchKernelGGL(k_emit_ellipse<uint32_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, splats, rects,
                           depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
      else
        hipLaunchKernelGGL(k_emit<uint32_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, rects, depths, n, order,
                           order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
    }
    // The 64-bit keys go to the key buffer the sorted tile ids do not end in, written by the last sort pass (or by
    // the range kernel when there is no pass).
    bool keys_done = !ctx->bin_keys;
    if (tile_bits > 0 && P > 0) {
      res = (sort_passes(tile_bits) & 1u) ? 1 : 0;  // odd pass count: result in buffer 1
      uint32_t* vr = static_cast<uint32_t*>(a.vals[res].ptr);
      uint32_t* vt = static_cast<uint32_t*>(a.vals[1 - res].ptr);
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, false);
      if (ctx->bin_keys) {
        // the last pass reads buffer 1 - res and writes buffer res; the 64-bit keys need a third place
        if ((st = grow(ctx, a.order_alt, std::max<size_t>(size_t(n) * 8, size_t(P) * 8)))) return st;
        final_k = static_cast<uint64_t*>(a.order_alt.ptr);
        st = radix_sort_tiles_final(ctx, s, kb[0], v0, P, tile_bits, kb[res], vr, kb[1 - res], vt, final_k, depths, n,
                                    pairs_dev);
        keys_done = true;
      } else {
        st = radix_sort_launch<uint32_t>(ctx, s, kb[0], v0, P, tile_bits, kb[res], vr, kb[1 - res], vt, pairs_dev);
      }
      if (st) return st;
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, true);
    }
    uint64_t* ranges_final = nullptr;
    if (!keys_done) final_k = ranges_final = static_cast<uint64_t*>(a.keys[1 - res].ptr);
    hipLaunchKernelGGL(k_ranges<uint32_t>, dim3(grid_for(P + 1, kThreads * kRangeItems)), dim3(kThreads), 0, s,
                       kb[res], static_cast<const uint32_t*>(a.vals[res].ptr), P, pairs_dev, uint32_t(num_tiles),
                       depths, n, ranges_final, ranges, 0u);
    sorted_v = static_cast<uint32_t*>(a.vals[res].ptr);
  } else {
    uint64_t* kb[2] = {static_cast<uint64_t*>(a.keys[0].ptr), static_cast<uint64_t*>(a.keys[1].ptr)};
    if (n)
    {
      if (ellipse)
        hipLaunchKernelGGL(k_emit_ellipse<uint64_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, splats, rects,
                           depths, n, order, order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
      else
        hipLaunchKernelGGL(k_emit<uint64_t>, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, rects, depths, n, order,
                           order_mask, tiles_x, offsets, P, pairs_dev, kb[0], v0, 0u);
    }
    if (P > 0) {
      const uint32_t key_bits = 32 + tile_bits;
      res = (sort_passes(key_bits) & 1u) ? 1 : 0;
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, false);
      st = radix_sort_launch<uint64_t>(ctx, s, kb[0], v0, P, key_bits, kb[res],
                                       static_cast<uint32_t*>(a.vals[res].ptr), kb[1 - res],
                                       static_cast<uint32_t*>(a.vals[1 - res].ptr), pairs_dev);
      if (st) return st;
      timing_mark(ctx, GSR_STAGE_TILE_SORT, s, true);
    }
    final_k = ctx->bin_keys ? kb[res] : nullptr;  // the sort's own keys, returned only when asked for
    hipLaunchKernelGGL(k_ranges<uint64_t>, dim3(grid_for(P + 1, kThreads * kRangeItems)), dim3(kThreads), 0, s,
                       kb[res], static_cast<const uint32_t*>(a.vals[res].ptr), P, pairs_dev, uint32_t(num_tiles),
                       depths, n, static_cast<uint64_t*>(nullptr), ranges, 0u);
    sorted_v = static_cast<uint32_t*>(a.vals[res].ptr);
  }
  timing_mark(ctx, GSR_STAGE_BIN, s, true);
  if ((st = check_launch(ctx, "gsr_bin emit/sort/ranges"))) return st;
  out->keys = final_k;
  out->vals = sorted_v;
  out->ranges = ranges;
  out->num_pairs = uint32_t(P);
  out->tiles_x = tiles_x;
  out->tiles_y = tiles_y;
  out->splat_pairs = n ? counts : nullptr;
  out->num_splats = n;
  return GSR_OK;
}

extern "C" gsr_status gsr_bin_pair_count(gsr_ctx* ctx, uint64_t* num_pairs, int32_t* overflowed) {
  if (!ctx || !num_pairs || !overflowed) return GSR_EINVAL;
  gsr_status st = enter(ctx);
  if (st) return st;
  if (ctx->pairs_pending) {
    const hipError_t e = hipEventSynchronize(ctx->arena.total_ready);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bin_pair_count");
    note_pair_count(ctx);
  }
  *num_pairs = ctx->last_pairs;
  *overflowed = ctx->last_pairs > ctx->last_cap ? 1 : 0;
  return GSR_OK;
}
