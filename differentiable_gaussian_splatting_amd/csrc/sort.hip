// Stable LSD radix sort of (key, uint32 value) pairs with 32- or 64-bit keys, 6- or 8-bit digits, for gfx950.
//
// One pass per non-constant digit, three launches per pass (reduce-then-scan, no inter-block waiting):
//   upsweep  each block of 256 x kItems keys counts its digits (per-wave LDS histograms);
//   scan     one workgroup per digit turns the per-block counts into global start positions;
//   scatter  each block ranks its keys stably with a 64-lane ballot match (the wave64 form of the simd-ballot
//            ranking of the pages' radix scatter), reorders them by digit in LDS, and writes each digit's run
//            contiguously.
// Digits above key_bits are identity passes of a stable sort and are never run (the constant-digit pass skip of
// the C0 resident arena + C1 pass skip page, section 2 table, row "C1"). Small sorts use 1024-key blocks so the
// grid still covers the 256 compute units; large ones 4096-key blocks.
//
// Packed form (binning's tile sort when the splat index and the tile id fit 32 bits together): each key is
// (tile << idx_bits) | splat, there is no separate value array, and the passes sort by the tile field only; the
// last pass unpacks the splat index into the value output (and the 64-bit keys when asked). Every pass then moves
// 4 bytes per pair instead of 8.
#include "gsr_internal.hpp"
#include "scan_common.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint64_t kSmallSort = uint64_t(1) << 21;  // below this many keys: 4 keys per thread, else 16
constexpr uint32_t kLargeItems = 16;  // 4096-key blocks: digit runs twice as long in the scatter's writes

template <uint32_t kBits, typename K>
__device__ __forceinline__ uint32_t digit_of(K k, uint32_t shift) {
  return uint32_t(k >> shift) & ((1u << kBits) - 1u);
}

// Digit counts of one block of keys. The order of the keys does not matter here, so each wave adds its keys to a
// histogram of its own with LDS atomics (a wave's atomics on one address serialise, different waves never share
// one), and the four are summed at the end.
template <typename K, uint32_t kItems, uint32_t kBits>
__global__ __launch_bounds__(kThreads) void k_upsweep(const K* __restrict__ keys, uint64_t n_cap,
                                                      const uint64_t* __restrict__ n_dev, uint32_t shift,
                                                      uint32_t nb, uint32_t* __restrict__ hist) {
  constexpr uint32_t kRadix = 1u << kBits, kWaves = kThreads / kWave;
  constexpr uint32_t kBlockKeys = kThreads * kItems, kWaveKeys = kWave * kItems;
  __shared__ uint32_t h[kWaves][kRadix];
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint64_t n = count_within(n_dev, n_cap);
  if (uint64_t(blockIdx.x) * kBlockKeys >= n) {  // a block past the keys counts nothing (its column stays in the scan)
    if (tid < kRadix) hist[uint64_t(tid) * nb + blockIdx.x] = 0;
    return;
  }
  for (uint32_t i = tid; i < kWaves * kRadix; i += kThreads) (&h[0][0])[i] = 0;
  const uint64_t base = uint64_t(blockIdx.x) * kBlockKeys + uint64_t(w) * kWaveKeys;
  // every load is issued before the first count (clamped indexes: no masked loads, no wait per key)
  K k[kItems];
#pragma unroll
  for (uint32_t i = 0; i < kItems; ++i) k[i] = keys[min(base + uint64_t(i) * kWave + lane, n - 1)];
  __syncthreads();
#pragma unroll
  for (uint32_t i = 0; i < kItems; ++i)
    if (base + uint64_t(i) * kWave + lane < n) atomicAdd(&h[w][digit_of<kBits>(k[i], shift)], 1u);
  __syncthreads();
  if (tid < kRadix) {
    uint32_t c = 0;
#pragma unroll
    for (uint32_t q = 0; q < kWaves; ++q) c += h[q][tid];
    hist[uint64_t(tid) * nb + blockIdx.x] = c;
  }
}

// Block d scans row d of hist (the counts of digit d in blocks 0..nb-1) in place; digit_tot[d] = row total.
__global__ __launch_bounds__(kThreads) void k_scan_rows(uint32_t* __restrict__ hist, uint32_t nb,
                                                        uint32_t* __restrict__ digit_tot) {
  __shared__ uint32_t smem[kThreads / kWave];
  uint32_t* row = hist + uint64_t(blockIdx.x) * nb;
  const uint32_t per = (nb + kThreads - 1) / kThreads;
  const uint32_t b0 = min(nb, threadIdx.x * per), b1 = min(nb, b0 + per);
  uint32_t sum = 0;
  for (uint32_t i = b0; i < b1; ++i) sum += row[i];
  uint32_t total;
  uint32_t run = block_exclusive_scan<uint32_t, kThreads>(sum, &total, smem);
  for (uint32_t i = b0; i < b1; ++i) {
    const uint32_t v = row[i];
    row[i] = run;
    run += v;
  }
  if (threadIdx.x == 0) digit_tot[blockIdx.x] = total;
}

// kFinal (32-bit tile ids, last pass): also writes keys_final[g] = (tile << 32) | bits(depths[value]) (when
// keys_final is not null). kPacked: keys are (tile << idx_bits) | value with no value array; a kFinal pass writes
// the unpacked values to vals_out, other passes write keys only.
template <typename K, uint32_t kItems, uint32_t kBits, bool kFinal, bool kPacked = false>
__global__ __launch_bounds__(kThreads) void k_scatter(const K* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
                                                      uint64_t n_cap, const uint64_t* __restrict__ n_dev,
                                                      uint32_t shift, uint32_t nb,
                                                      const uint32_t* __restrict__ hist,
                                                      const uint32_t* __restrict__ digit_tot, K* __restrict__ keys_out,
                                                      uint32_t* __restrict__ vals_out,
                                                      uint64_t* __restrict__ keys_final,
                                                      const float* __restrict__ depths, uint32_t n_depths,
                                                      uint32_t idx_bits) {
  constexpr uint32_t kRadix = 1u << kBits, kWaves = kThreads / kWave;
  constexpr uint32_t kBlockKeys = kThreads * kItems, kWaveKeys = kWave * kItems;
  __shared__ K s_keys[kBlockKeys];
  __shared__ uint32_t s_vals[kPacked ? 1 : kBlockKeys];
  __shared__ uint32_t s_wave[kWaves][kRadix];  // per-wave running digit counts, then wave prefixes
  __shared__ uint32_t s_dstart[kRadix];        // first LDS slot of each digit in this block
  __shared__ uint32_t s_gbase[kRadix];         // global position of this block's first key of each digit
  __shared__ uint32_t smem[kWaves];
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint64_t n = count_within(n_dev, n_cap);
  if (uint64_t(blockIdx.x) * kBlockKeys >= n) return;

  // all key and value loads are issued first (clamped indexes, no masked loads), so their latency overlaps the
  // block's scan of the digit bases below
  K k[kItems];
  uint32_t v[kItems], r[kItems];
  const uint64_t base = uint64_t(blockIdx.x) * kBlockKeys + uint64_t(w) * kWaveKeys;
#pragma unroll
  for (uint32_t i = 0; i < kItems; ++i) {
    const uint64_t idx = min(base + uint64_t(i) * kWave + lane, n - 1);
    k[i] = keys_in[idx];
    if constexpr (!kPacked) v[i] = vals_in[idx];
  }
  for (uint32_t i = tid; i < kWaves * kRadix; i += kThreads) (&s_wave[0][0])[i] = 0;
  {
    const uint32_t dbase = block_exclusive_scan<uint32_t, kThreads>(tid < kRadix ? digit_tot[tid] : 0u, nullptr,
                                                                     smem);
    if (tid < kRadix) s_gbase[tid] = dbase + hist[uint64_t(tid) * nb + blockIdx.x];
  }
  __syncthreads();

#pragma unroll
  for (uint32_t i = 0; i < kItems; ++i) {
    const bool valid = base + uint64_t(i) * kWave + lane < n;
    const uint32_t d = digit_of<kBits>(k[i], shift);
    const uint64_t peers = match_digit<kBits>(d, valid);
    r[i] = 0;
    if (valid) {
      const uint64_t before = peers & lanemask_lt(lane);
      const uint32_t old = s_wave[w][d];
      r[i] = old + uint32_t(__popcll(before));
      if (before == 0) s_wave[w][d] = old + uint32_t(__popcll(peers));
    }
  }
  __syncthreads();
  {
    // thread tid < kRadix owns digit tid: wave prefixes in place, and the digit's first slot in the block
    uint32_t run = 0;
    if (tid < kRadix) {
#pragma unroll
      for (uint32_t q = 0; q < kWaves; ++q) {
        const uint32_t c = s_wave[q][tid];
        s_wave[q][tid] = run;
        run += c;
      }
    }
    const uint32_t ds = block_exclusive_scan<uint32_t, kThreads>(run, nullptr, smem);
    if (tid < kRadix) s_dstart[tid] = ds;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t i = 0; i < kItems; ++i) {
    const uint64_t idx = base + uint64_t(i) * kWave + lane;
    if (idx < n) {
      const uint32_t d = digit_of<kBits>(k[i], shift);
      const uint32_t pos = s_dstart[d] + s_wave[w][d] + r[i];
      s_keys[pos] = k[i];
      if constexpr (!kPacked) s_vals[pos] = v[i];
    }
  }
  __syncthreads();
  const uint64_t block0 = uint64_t(blockIdx.x) * kBlockKeys;
  const uint32_t count = uint32_t(min<uint64_t>(kBlockKeys, n - block0));
  for (uint32_t j = tid; j < count; j += kThreads) {
    const K kk = s_keys[j];
    const uint32_t d = digit_of<kBits>(kk, shift);
    const uint64_t g = uint64_t(s_gbase[d]) + (j - s_dstart[d]);
    if (g < n) {  // always true for consistent counts; keeps a miscount from writing out of bounds
      keys_out[g] = kk;
      if constexpr (kPacked) {
        if constexpr (kFinal) {
          const uint32_t val = uint32_t(kk) & ((1u << idx_bits) - 1u);
          vals_out[g] = val;
          if (keys_final)
            keys_final[g] = (uint64_t(uint32_t(kk) >> idx_bits) << 32) |
                            (val < n_depths ? __float_as_uint(depths[val]) : 0u);
        }
      } else {
        const uint32_t val = s_vals[j];
        vals_out[g] = val;
        if constexpr (kFinal)
          keys_final[g] = (uint64_t(kk) << 32) | (val < n_depths ? __float_as_uint(depths[val]) : 0u);
      }
    }
  }
}

struct FinalKeys {
  uint64_t* keys = nullptr;
  const float* depths = nullptr;
  uint32_t n = 0;
  bool packed = false;    // keys are (tile << idx_bits) | value; vals_in is unused
  uint32_t idx_bits = 0;  // packed: width of the value field, which the passes skip
};

template <typename K, uint32_t kItems, uint32_t kBits>
gsr_status run_passes(gsr_ctx* ctx, hipStream_t s, const K* keys_in, const uint32_t* vals_in, uint64_t n,
                      const uint64_t* n_dev, uint32_t passes, K* keys_out, uint32_t* vals_out, K* tmp_keys,
                      uint32_t* tmp_vals, FinalKeys fin) {
  constexpr uint32_t kRadix = 1u << kBits;
  const uint32_t nb = uint32_t((n + kThreads * kItems - 1) / (kThreads * kItems));
  gsr_status st = grow(ctx, ctx->arena.hist, size_t(nb) * kRadix * 4);
  if (st) return st;
  if ((st = grow(ctx, ctx->arena.digit_tot, kRadix * 4))) return st;
  uint32_t* hist = static_cast<uint32_t*>(ctx->arena.hist.ptr);
  uint32_t* tot = static_cast<uint32_t*>(ctx->arena.digit_tot.ptr);
  const K* src_k = keys_in;
  const uint32_t* src_v = vals_in;
  for (uint32_t p = 0; p < passes; ++p) {
    const bool to_out = ((passes - p) & 1u) == 1u;
    K* dk = to_out ? keys_out : tmp_keys;
    uint32_t* dv = to_out ? vals_out : tmp_vals;
    if (p == 0 && dk == keys_in) return fail(ctx, GSR_EINVAL, "radix sort: first pass would overwrite its input");
    const uint32_t shift = fin.idx_bits + kBits * p;
    hipLaunchKernelGGL((k_upsweep<K, kItems, kBits>), dim3(nb), dim3(kThreads), 0, s, src_k, n, n_dev, shift, nb,
                       hist);
    hipLaunchKernelGGL(k_scan_rows, dim3(kRadix), dim3(kThreads), 0, s, hist, nb, tot);
    const bool last = p + 1 == passes;
    if constexpr (sizeof(K) == 4) {
      if (fin.packed) {
        // keys only; the last pass unpacks the values (into vals_out, which the caller sized), if asked to
        if (last && vals_out)
          hipLaunchKernelGGL((k_scatter<K, kItems, kBits, true, true>), dim3(nb), dim3(kThreads), 0, s, src_k,
                             static_cast<const uint32_t*>(nullptr), n, n_dev, shift, nb, hist, tot, dk, vals_out,
                             fin.keys, fin.depths, fin.n, fin.idx_bits);
        else
          hipLaunchKernelGGL((k_scatter<K, kItems, kBits, false, true>), dim3(nb), dim3(kThreads), 0, s, src_k,
                             static_cast<const uint32_t*>(nullptr), n, n_dev, shift, nb, hist, tot, dk,
                             static_cast<uint32_t*>(nullptr), static_cast<uint64_t*>(nullptr),
                             static_cast<const float*>(nullptr), 0u, fin.idx_bits);
        src_k = dk;
        continue;
      }
    }
    bool final_pass = false;
    if constexpr (sizeof(K) == 4) final_pass = fin.keys && last;
    if (final_pass)
      hipLaunchKernelGGL((k_scatter<K, kItems, kBits, true>), dim3(nb), dim3(kThreads), 0, s, src_k, src_v, n, n_dev,
                         shift, nb, hist, tot, dk, dv, fin.keys, fin.depths, fin.n, 0u);
    else
      hipLaunchKernelGGL((k_scatter<K, kItems, kBits, false>), dim3(nb), dim3(kThreads), 0, s, src_k, src_v, n, n_dev,
                         shift, nb, hist, tot, dk, dv, static_cast<uint64_t*>(nullptr),
                         static_cast<const float*>(nullptr), 0u, 0u);
    src_k = dk;
    src_v = dv;
  }
  return check_launch(ctx, "radix sort");
}

// Keys of up to 12 significant bits take 6-bit digits (64 buckets: longer runs per block in the scatter and
// fewer ballots per key), longer keys 8-bit digits.
constexpr uint32_t kNarrowKeyBits = 12;

}  // namespace

uint32_t sort_blocks(uint64_t n) {
  const uint64_t per = kThreads * (n < kSmallSort ? 4u : kLargeItems);
  return uint32_t((n + per - 1) / per);
}

uint32_t sort_passes(uint32_t key_bits) {
  return key_bits <= kNarrowKeyBits ? (key_bits + 5) / 6 : (key_bits + 7) / 8;
}

// Pass p writes to keys_out when (passes - p) is odd and to tmp otherwise, so the last pass lands in keys_out.
// The first destination must differ from keys_in: with an even pass count keys_in may be keys_out, with an odd
// one keys_in may be tmp.
namespace {
// With n_dev, n is a capacity and the launches sort *n_dev keys (none when *n_dev > n).
template <typename K>
gsr_status sort_any(gsr_ctx* ctx, hipStream_t s, const K* keys_in, const uint32_t* vals_in, uint64_t n,
                    const uint64_t* n_dev, uint32_t key_bits, K* keys_out, uint32_t* vals_out, K* tmp_keys,
                    uint32_t* tmp_vals, FinalKeys fin) {
  if (n == 0) return GSR_OK;
  const uint32_t passes = sort_passes(key_bits);
  if (key_bits <= kNarrowKeyBits) {
    if (n < kSmallSort)
      return run_passes<K, 4, 6>(ctx, s, keys_in, vals_in, n, n_dev, passes, keys_out, vals_out, tmp_keys, tmp_vals,
                                 fin);
    return run_passes<K, kLargeItems, 6>(ctx, s, keys_in, vals_in, n, n_dev, passes, keys_out, vals_out, tmp_keys,
                                         tmp_vals, fin);
  }
  if (n < kSmallSort)
    return run_passes<K, 4, 8>(ctx, s, keys_in, vals_in, n, n_dev, passes, keys_out, vals_out, tmp_keys, tmp_vals,
                               fin);
  return run_passes<K, kLargeItems, 8>(ctx, s, keys_in, vals_in, n, n_dev, passes, keys_out, vals_out, tmp_keys,
                                       tmp_vals, fin);
}
}  // namespace

template <typename K>
gsr_status radix_sort_launch(gsr_ctx* ctx, hipStream_t s, const K* keys_in, const uint32_t* vals_in, uint64_t n,
                             uint32_t key_bits, K* keys_out, uint32_t* vals_out, K* tmp_keys, uint32_t* tmp_vals,
                             const uint64_t* n_dev) {
  return sort_any<K>(ctx, s, keys_in, vals_in, n, n_dev, key_bits, keys_out, vals_out, tmp_keys, tmp_vals,
                     FinalKeys{});
}

gsr_status radix_sort_tiles_final(gsr_ctx* ctx, hipStream_t s, const uint32_t* keys_in, const uint32_t* vals_in,
                                  uint64_t n, uint32_t key_bits, uint32_t* keys_out, uint32_t* vals_out,
                                  uint32_t* tmp_keys, uint32_t* tmp_vals, uint64_t* keys_final,
                                  const float* depths, uint32_t n_depths, const uint64_t* n_dev) {
  if (key_bits == 0) return fail(ctx, GSR_EINVAL, "radix sort: final keys need at least one pass");
  return sort_any<uint32_t>(ctx, s, keys_in, vals_in, n, n_dev, key_bits, keys_out, vals_out, tmp_keys, tmp_vals,
                            FinalKeys{keys_final, depths, n_depths});
}

gsr_status radix_sort_tiles_packed(gsr_ctx* ctx, hipStream_t s, const uint32_t* keys_in, uint64_t n,
                                   uint32_t idx_bits, uint32_t tile_bits, uint32_t* keys_out, uint32_t* tmp_keys,
                                   uint32_t* vals_out, uint64_t* keys_final, const float* depths,
                                   uint32_t n_depths, const uint64_t* n_dev) {
  if (tile_bits == 0 || idx_bits + tile_bits > 32)
    return fail(ctx, GSR_EINVAL, "radix sort: packed keys need 1..32 - idx_bits tile bits");
  if (!vals_out && keys_final) return fail(ctx, GSR_EINVAL, "radix sort: final keys need the value output");
  FinalKeys fin{keys_final, depths, n_depths, true, idx_bits};
  return sort_any<uint32_t>(ctx, s, keys_in, nullptr, n, n_dev, tile_bits, keys_out, vals_out, tmp_keys, nullptr,
                            fin);
}

template gsr_status radix_sort_launch<uint32_t>(gsr_ctx*, hipStream_t, const uint32_t*, const uint32_t*, uint64_t,
                                                uint32_t, uint32_t*, uint32_t*, uint32_t*, uint32_t*,
                                                const uint64_t*);
template gsr_status radix_sort_launch<uint64_t>(gsr_ctx*, hipStream_t, const uint64_t*, const uint32_t*, uint64_t,
                                                uint32_t, uint64_t*, uint32_t*, uint64_t*, uint32_t*,
                                                const uint64_t*);

}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_radix_sort(gsr_ctx* ctx, void* stream, const uint64_t* keys_in, const uint32_t* vals_in,
                                     uint64_t n, uint32_t key_bits, uint64_t* keys_out, uint32_t* vals_out) {
  if (!ctx) return GSR_EINVAL;
  if (key_bits == 0 || key_bits > 64) return fail(ctx, GSR_EINVAL, "gsr_radix_sort: key_bits must be in 1..64");
  if (n >= (uint64_t(1) << 32)) return fail(ctx, GSR_EOVERFLOW, "gsr_radix_sort: n >= 2^32");
  if (n == 0) return GSR_OK;
  if (!keys_in || !vals_in || !keys_out || !vals_out)
    return fail(ctx, GSR_EINVAL, "gsr_radix_sort: null pointer");
  const uint64_t lo_in = reinterpret_cast<uintptr_t>(keys_in), lo_out = reinterpret_cast<uintptr_t>(keys_out);
  if (lo_in < lo_out + n * 8 && lo_out < lo_in + n * 8)
    return fail(ctx, GSR_EINVAL, "gsr_radix_sort: keys_in and keys_out overlap");
  gsr_status st = enter(ctx);
  if (st) return st;
  Arena& a = ctx->arena;
  if ((st = grow(ctx, a.keys[0], size_t(n) * 8)) || (st = grow(ctx, a.vals[0], size_t(n) * 4))) return st;
  return radix_sort_launch<uint64_t>(ctx, static_cast<hipStream_t>(stream), keys_in, vals_in, n, key_bits, keys_out,
                                     vals_out, static_cast<uint64_t*>(a.keys[0].ptr),
                                     static_cast<uint32_t*>(a.vals[0].ptr));
}
