// Depth order within tiles for the tile-first binning scheme (GSR_BIN_TILE_DEPTH): the order of the 64-bit keys
// (tile << 32) | depth bits sorted stably, ties in depth keeping splat order. [C0 resident arena + C1 pass skip page,
// section 2 table, rows "C0" and "C1": the keys and their stable sort; the constant-digit pass skip is applied per
// list] Two forms. The per-tile order: the pairs have been put in tile order (emitted splat by splat and sorted
// stably by tile id, or by a counting sort), and one workgroup per tile puts the tile's list in (depth bits, splat
// index) order. The per-super-tile order (below): the counting sort filled the lists of squares of 2 x 2 tiles,
// and one workgroup per square sorts its list once and filters it into its four tiles' lists.
//
// Lists of at most kCap entries are sorted in LDS by buckets: the pair (depth bits, splat) is unique within a tile
// (a splat covers a tile once), so the sort needs no stability. Each entry goes to one of nb buckets (nb = the
// power of two >= the list length, 512 to 4096) by a monotone map of its depth bits, (bits - min) * nb / (max - min
// + 1) in fp32 with truncation; a counting sort by bucket (LDS atomics give each entry a slot in its bucket in no
// particular order) groups them, and each entry's rank in the tile is its bucket's start plus the number of entries
// of its bucket with a smaller (depth bits, splat). On the pages' depth distributions a bucket holds about three
// entries; a tile with a bucket of more than kBucketLimit (many equal depths) takes the radix sort instead.
//
// The radix sort is a least-significant-digit sort of the list's 32-bit depth keys in 8-bit digits, in LDS when the
// list has at most kCap entries (keys and 16-bit positions in the tile's list, double-buffered), else in the same
// steps through global scratch. Per pass: a digit histogram of the whole list (per-wave LDS counts), its exclusive
// scan, and a stable scatter of chunks of 1024 keys in list order, each key ranked among the equal digits of its
// wave by a 64-lane ballot match (as the device-wide sort's scatter) and placed after those of earlier waves and
// chunks. A pass whose digit is the same for every key of the list is skipped. Being stable, it needs the list in
// splat order for the ties: a list in any other order (the fused counting sort by tile places each block's pairs in
// no particular order within its stretch of the tile's list) is first sorted by splat index, the same way.
#include "gsr_internal.hpp"
#include "scan_common.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 512, kWaves = kThreads / kWave;
constexpr uint32_t kBits = 8, kRadix = 1u << kBits;
constexpr uint32_t kItems = 4, kChunk = kThreads * kItems;  // keys ranked per step, four per thread
constexpr uint32_t kCap = 3456;  // the longest list sorted in LDS (52 KB per workgroup: three per compute unit)
static_assert(kThreads >= kRadix, "a thread per digit");
static_assert(kCap <= 65536, "16-bit list positions");
constexpr uint32_t kMinBuckets = kThreads, kMaxBuckets = 4096;  // kMaxBuckets: kCap rounded up to a power of two
constexpr uint32_t kBucketLimit = 64;
constexpr uint32_t kMaxItems = (kCap + kThreads - 1) / kThreads;  // list entries per thread
constexpr uint32_t kScanPer = kMaxBuckets / kThreads;             // bucket counts per thread in the scan
static_assert(kMaxBuckets >= kCap && kMinBuckets >= kThreads && kMaxBuckets % kThreads == 0, "bucket counts");

struct SortShared {
  uint32_t hist[kWaves][kRadix];  // per-wave digit counts, then per-wave prefixes within a chunk
  uint32_t dstart[kRadix];        // first position of each digit in the pass's output
  uint32_t run[kRadix];           // keys of each digit placed by the earlier chunks
  uint32_t tot[kRadix];           // keys of each digit in the current chunk
  uint32_t smem[kWaves];
};

union TileShared {
  struct {
    SortShared sh;
    uint32_t key[2][kCap];
    uint16_t pos[2][kCap];
  } lsd;
  struct {
    uint32_t start[kMaxBuckets + 1];  // bucket counts, then their exclusive scan; start[nb] = m
    uint64_t entry[kCap];             // the list grouped by bucket: (depth bits << 32) | splat
    uint32_t wmin[kWaves], wmax[kWaves], wsum[kWaves];
  } bkt;
  struct {                            // lists longer than kCap: the entries go through the arena
    uint32_t start[kMaxBuckets + 1];
    uint32_t run[kMaxBuckets];        // next free slot of each bucket
    uint32_t wmin[kWaves], wmax[kWaves], wsum[kWaves];
  } big;
};

__device__ __forceinline__ uint32_t bucket_of(uint32_t key, uint32_t lo, float scale, uint32_t nb) {
  return min(nb - 1, uint32_t(float(key - lo) * scale));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int d = 1; d < int(kWave); d <<= 1) v = min(v, uint32_t(__shfl_xor(int(v), d)));
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 1; d < int(kWave); d <<= 1) v = max(v, uint32_t(__shfl_xor(int(v), d)));
  return v;
}

// Sorts keys k0[0..m) with their positions p0[0..m) stably by the keys' 32 bits, through (k1, p1); returns which
// buffer pair holds the result (0 or 1). The buffers are LDS (short lists) or global scratch (long ones). All threads
// call it.
template <typename PosT>
__device__ __forceinline__ uint32_t sort_list(uint32_t* k0, uint32_t* k1, PosT* p0, PosT* p1, uint32_t m,
                                              SortShared& sh) {
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const bool owner = tid < kRadix;  // thread tid < kRadix owns digit tid
  uint32_t src = 0;
  for (uint32_t shift = 0; shift < 32; shift += kBits) {
    uint32_t* const ks = src ? k1 : k0;
    uint32_t* const kd = src ? k0 : k1;
    PosT* const ps = src ? p1 : p0;
    PosT* const pd = src ? p0 : p1;
    for (uint32_t i = tid; i < kWaves * kRadix; i += kThreads) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < m; e += kThreads) atomicAdd(&sh.hist[w][(ks[e] >> shift) & (kRadix - 1)], 1u);
    __syncthreads();
    uint32_t tot = 0;
    if (owner) {
#pragma unroll
      for (uint32_t q = 0; q < kWaves; ++q) tot += sh.hist[q][tid];
    }
    // one digit holding every key: this pass is the identity (uniform)
    if (__syncthreads_or(owner && tot == m)) continue;
    const uint32_t ds = block_exclusive_scan<uint32_t, kThreads>(tot, nullptr, sh.smem);
    if (owner) {
      sh.dstart[tid] = ds;
      sh.run[tid] = 0;
    }
    for (uint32_t c0 = 0; c0 < m; c0 += kChunk) {
      for (uint32_t i = lane; i < kRadix; i += kWave) sh.hist[w][i] = 0;
      __syncthreads();
      uint32_t kk[kItems], d[kItems], r[kItems];
      PosT pp[kItems];
      bool valid[kItems];
#pragma unroll
      for (uint32_t i = 0; i < kItems; ++i) {
        const uint32_t idx = c0 + w * (kWave * kItems) + i * kWave + lane;
        valid[i] = idx < m;
        kk[i] = valid[i] ? ks[idx] : 0u;
        pp[i] = valid[i] ? ps[idx] : PosT(0);
        d[i] = (kk[i] >> shift) & (kRadix - 1);
        const uint64_t peers = match_digit<kBits>(d[i], valid[i]);
        r[i] = 0;
        if (valid[i]) {
          const uint64_t before = peers & lanemask_lt(lane);
          const uint32_t old = sh.hist[w][d[i]];
          r[i] = old + uint32_t(__popcll(before));
          if (before == 0) sh.hist[w][d[i]] = old + uint32_t(__popcll(peers));
        }
      }
      __syncthreads();
      if (owner) {
        uint32_t acc = 0;  // per-wave prefixes of digit tid and the chunk's total
#pragma unroll
        for (uint32_t q = 0; q < kWaves; ++q) {
          const uint32_t c = sh.hist[q][tid];
          sh.hist[q][tid] = acc;
          acc += c;
        }
        sh.tot[tid] = acc;
      }
      __syncthreads();
#pragma unroll
      for (uint32_t i = 0; i < kItems; ++i)
        if (valid[i]) {
          const uint32_t dst = sh.dstart[d[i]] + sh.run[d[i]] + sh.hist[w][d[i]] + r[i];
          kd[dst] = kk[i];
          pd[dst] = pp[i];
        }
      __syncthreads();
      if (owner) sh.run[tid] += sh.tot[tid];
    }
    __syncthreads();
    src = 1 - src;
  }
  return src;
}

// The list's positions in (depth bits, splat) order with their depth bits, through the buffer pairs (k0, p0) and
// (k1, p1); returns which pair holds them. Unless the list is in splat order, it is first sorted by splat index
// (unique keys), and the depth sort then runs on that order.
template <typename PosT, typename SplatAt, typename DepthBits>
__device__ __forceinline__ uint32_t radix_order(uint32_t* k0, uint32_t* k1, PosT* p0, PosT* p1, uint32_t m,
                                                bool ordered, SplatAt splat_at, DepthBits depth_bits,
                                                SortShared& sh) {
  const uint32_t tid = threadIdx.x;
  uint32_t r = 0;
  if (!ordered) {
    for (uint32_t e = tid; e < m; e += kThreads) {
      k0[e] = splat_at(e);
      p0[e] = PosT(e);
    }
    __syncthreads();
    r = sort_list(k0, k1, p0, p1, m, sh);
  } else {
    for (uint32_t e = tid; e < m; e += kThreads) p0[e] = PosT(e);
  }
  uint32_t* const ka = r ? k1 : k0;
  uint32_t* const kb = r ? k0 : k1;
  PosT* const pa = r ? p1 : p0;
  PosT* const pb = r ? p0 : p1;
  for (uint32_t e = tid; e < m; e += kThreads) ka[e] = depth_bits(splat_at(pa[e]));
  __syncthreads();
  return sort_list(ka, kb, pa, pb, m, sh) ? 1 - r : r;
}

// Exclusive scan of the bucket counts start[0..nb) in place (nb a multiple of kThreads, at most kMaxBuckets;
// start[nb] = m); returns the largest count. All threads call it; it ends with a barrier.
__device__ __forceinline__ uint32_t scan_buckets(uint32_t* start, uint32_t nb, uint32_t m, uint32_t* wsum) {
  const uint32_t tid = threadIdx.x, per = nb / kThreads;
  uint32_t c[kScanPer], sum = 0, biggest = 0;
#pragma unroll
  for (uint32_t j = 0; j < kScanPer; ++j) {
    c[j] = j < per ? start[tid * per + j] : 0u;
    sum += c[j];
    biggest = max(biggest, c[j]);
  }
  uint32_t run = block_exclusive_scan<uint32_t, kThreads>(sum, nullptr, wsum);
#pragma unroll
  for (uint32_t j = 0; j < kScanPer; ++j)
    if (j < per) {
      start[tid * per + j] = run;
      run += c[j];
    }
  if (tid == 0) start[nb] = m;
  __syncthreads();
  return biggest;
}

// One tile, by one workgroup. The tile's list is list[start..end) (ranges, clamped to the pair count): packed words
// (tile << idx_bits) | splat when list_vals is null, else list_vals holds the splats; `ordered` says the list is in
// ascending splat order. Writes vals_out[start + e] = the e-th splat in (depth bits, index) order and, when keys_out
// is not null, keys_out[start + e] = (tile << 32) | its depth bits. Lists longer than kCap use the arena: the bucket
// path stages each entry's depth bits in gp0 and groups the entries (64-bit) in gent; the radix path the arrays gk0,
// gk1, gp0, gp1 (P entries each, every tile using its own stretch [start, end)). gent overlaps none of the four.
#define GSR_TILE_DEPTH_PARAMS                                                                                     \
  const uint32_t *__restrict__ list, const uint32_t *__restrict__ list_vals, uint32_t idx_bits, bool ordered,       \
      const uint32_t *__restrict__ ranges, uint64_t pairs_cap, const uint64_t *__restrict__ pairs_dev,             \
      uint32_t num_tiles, const float *__restrict__ depths, uint32_t n, uint32_t *__restrict__ vals_out,           \
      uint64_t *__restrict__ keys_out, uint64_t *gent, uint32_t *gk0, uint32_t *gk1, uint32_t *gp0, uint32_t *gp1

__device__ __forceinline__ void order_tile(uint32_t tile, TileShared& ts, GSR_TILE_DEPTH_PARAMS) {
  const uint64_t P = count_within(pairs_dev, pairs_cap);
  const uint32_t start = uint32_t(min<uint64_t>(ranges[2 * tile], P));
  const uint32_t end = uint32_t(max<uint64_t>(start, min<uint64_t>(ranges[2 * tile + 1], P)));
  const uint32_t m = end - start;
  if (m == 0) return;
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint32_t mask = idx_bits >= 32 ? ~0u : (1u << idx_bits) - 1u;
  auto splat_at = [&](uint32_t e) -> uint32_t { return list_vals ? list_vals[start + e] : list[start + e] & mask; };
  auto depth_bits = [&](uint32_t splat) -> uint32_t { return splat < n ? __float_as_uint(depths[splat]) : 0u; };
  // the results are written once and not read again here: non-temporal stores (4.5 us of 60 at 410k). The scatter
  // that fills the lists needs the opposite: its scattered 4-byte stores rely on merging in L2 (with non-temporal
  // stores it took 0.28 ms instead of 0.05).
  auto emit = [&](uint32_t e, uint32_t splat, uint32_t key) {
    __builtin_nontemporal_store(splat, &vals_out[start + e]);
    if (keys_out) __builtin_nontemporal_store((uint64_t(tile) << 32) | key, &keys_out[start + e]);
  };
  if (m <= kCap) {
    // buckets
    uint32_t key[kMaxItems], spl[kMaxItems], slot[kMaxItems];
    uint32_t kmin = ~0u, kmax = 0;
#pragma unroll
    for (uint32_t i = 0; i < kMaxItems; ++i) {
      const uint32_t e = tid + i * kThreads;
      spl[i] = e < m ? splat_at(e) : 0u;
      key[i] = e < m ? depth_bits(spl[i]) : 0u;
      if (e < m) kmin = min(kmin, key[i]), kmax = max(kmax, key[i]);
    }
    const uint32_t nb = max(kMinBuckets, 1u << (32 - __clz(int(m - 1))));
    for (uint32_t j = tid; j <= nb; j += kThreads) ts.bkt.start[j] = 0;
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) ts.bkt.wmin[w] = kmin, ts.bkt.wmax[w] = kmax;
    __syncthreads();
    uint32_t lo = ts.bkt.wmin[0], hi = ts.bkt.wmax[0];
#pragma unroll
    for (uint32_t q = 1; q < kWaves; ++q) lo = min(lo, ts.bkt.wmin[q]), hi = max(hi, ts.bkt.wmax[q]);
    const float scale = float(nb) / (float(hi - lo) + 1.0f);
#pragma unroll
    for (uint32_t i = 0; i < kMaxItems; ++i)
      if (tid + i * kThreads < m) slot[i] = atomicAdd(&ts.bkt.start[bucket_of(key[i], lo, scale, nb)], 1u);
    __syncthreads();
    // exclusive scan of the counts: thread tid takes nb / kThreads consecutive buckets
    const uint32_t biggest = scan_buckets(ts.bkt.start, nb, m, ts.bkt.wsum);
    if (!__syncthreads_or(biggest > kBucketLimit)) {
#pragma unroll
      for (uint32_t i = 0; i < kMaxItems; ++i)
        if (tid + i * kThreads < m)
          ts.bkt.entry[ts.bkt.start[bucket_of(key[i], lo, scale, nb)] + slot[i]] = (uint64_t(key[i]) << 32) | spl[i];
      __syncthreads();
      for (uint32_t q = tid; q < m; q += kThreads) {
        const uint64_t me = ts.bkt.entry[q];
        const uint32_t k = uint32_t(me >> 32);
        const uint32_t b = bucket_of(k, lo, scale, nb);
        const uint32_t b0 = ts.bkt.start[b], b1 = ts.bkt.start[b + 1];
        uint32_t r = b0;
        for (uint32_t f = b0; f < b1; ++f) r += ts.bkt.entry[f] < me ? 1u : 0u;
        emit(r, uint32_t(me), k);
      }
      return;
    }
    // a crowded bucket: the radix sort (the barrier above ends every read of the bucket layout)
    const uint32_t res = radix_order(ts.lsd.key[0], ts.lsd.key[1], ts.lsd.pos[0], ts.lsd.pos[1], m, ordered, splat_at,
                                     depth_bits, ts.lsd.sh);
    const uint32_t* kr = res ? ts.lsd.key[1] : ts.lsd.key[0];
    const uint16_t* pr = res ? ts.lsd.pos[1] : ts.lsd.pos[0];
    for (uint32_t e = tid; e < m; e += kThreads) emit(e, splat_at(pr[e]), kr[e]);
  } else {
    // buckets as above with kMaxBuckets of them; the depth bits staged in list order (one gather), the grouped
    // entries in the arena
    uint32_t* const staged = gp0 + start;
    uint32_t kmin = ~0u, kmax = 0;
    for (uint32_t e = tid; e < m; e += kThreads) {
      const uint32_t k = depth_bits(splat_at(e));
      staged[e] = k;
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
    const uint32_t nb = kMaxBuckets;
    for (uint32_t j = tid; j <= nb; j += kThreads) ts.big.start[j] = 0;
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) ts.big.wmin[w] = kmin, ts.big.wmax[w] = kmax;
    __syncthreads();
    uint32_t lo = ts.big.wmin[0], hi = ts.big.wmax[0];
#pragma unroll
    for (uint32_t q = 1; q < kWaves; ++q) lo = min(lo, ts.big.wmin[q]), hi = max(hi, ts.big.wmax[q]);
    const float scale = float(nb) / (float(hi - lo) + 1.0f);
    for (uint32_t e = tid; e < m; e += kThreads) atomicAdd(&ts.big.start[bucket_of(staged[e], lo, scale, nb)], 1u);
    __syncthreads();
    const uint32_t biggest = scan_buckets(ts.big.start, nb, m, ts.big.wsum);
    // a bucket may hold a few times the mean of m / nb entries before the radix sort is cheaper
    const uint32_t limit = max(kBucketLimit, 8 * ((m + nb - 1) / nb));
    if (!__syncthreads_or(biggest > limit)) {
      uint64_t* const ent = gent + start;
      for (uint32_t j = tid; j < nb; j += kThreads) ts.big.run[j] = ts.big.start[j];
      __syncthreads();
      for (uint32_t e = tid; e < m; e += kThreads) {
        const uint32_t k = staged[e];
        ent[atomicAdd(&ts.big.run[bucket_of(k, lo, scale, nb)], 1u)] = (uint64_t(k) << 32) | splat_at(e);
      }
      __syncthreads();
      for (uint32_t q = tid; q < m; q += kThreads) {
        const uint64_t me = ent[q];
        const uint32_t k = uint32_t(me >> 32);
        const uint32_t b = bucket_of(k, lo, scale, nb);
        const uint32_t b0 = ts.big.start[b], b1 = ts.big.start[b + 1];
        uint32_t r = b0;
        for (uint32_t f = b0; f < b1; ++f) r += ent[f] < me ? 1u : 0u;
        emit(r, uint32_t(me), k);
      }
      return;
    }
    uint32_t *k0 = gk0 + start, *k1 = gk1 + start, *p0 = gp0 + start, *p1 = gp1 + start;
    const uint32_t res = radix_order(k0, k1, p0, p1, m, ordered, splat_at, depth_bits, ts.lsd.sh);
    const uint32_t* kr = res ? k1 : k0;
    const uint32_t* pr = res ? p1 : p0;
    for (uint32_t e = tid; e < m; e += kThreads) emit(e, splat_at(pr[e]), kr[e]);
  }
}

// A workgroup per tile; past kMaxGrid tiles (a workgroup per tile of a 2^23-tile image would be 2^32 work-items,
// more than a launch takes) kLoop: workgroup b orders tiles b, b + gridDim.x, ...
constexpr uint32_t kMaxGrid = 1u << 20;

template <bool kLoop>
__global__ __launch_bounds__(kThreads) void k_tile_depth(GSR_TILE_DEPTH_PARAMS) {
  __shared__ TileShared ts;
  if constexpr (!kLoop) {
    if (blockIdx.x < num_tiles)
      order_tile(blockIdx.x, ts, list, list_vals, idx_bits, ordered, ranges, pairs_cap, pairs_dev, num_tiles, depths,
                 n, vals_out, keys_out, gent, gk0, gk1, gp0, gp1);
  } else {
    for (uint32_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
      order_tile(tile, ts, list, list_vals, idx_bits, ordered, ranges, pairs_cap, pairs_dev, num_tiles, depths, n,
                 vals_out, keys_out, gent, gk0, gk1, gp0, gp1);
      __syncthreads();  // the next tile reuses the LDS
    }
  }
}

// ---------------------------------------------------------------------------------------------------------------
// Per-super-tile order (the fused counting sort's second level). A super-tile is a square of 2 x 2 tiles; its list
// holds an entry (depth bits << 32) | (cover << 28) | splat for every splat whose tile rectangle meets it, in no
// particular order, cover being the four bits (2 dy + dx) of the tiles the rectangle covers. One workgroup sorts
// the list by (depth bits, splat) once - buckets in LDS as above (linear in the depth value rather than in its
// bits), or the radix sort through the arena for lists
// longer than kSupCap or with a crowded bucket - and then writes each of its tiles' lists by a stable filter of that
// order: an entry goes to tile j when its cover bit j is set. The cover bits follow the rule by which the tiles'
// totals (and so the ranges) were counted, so each tile's list comes out whole and in (depth bits, splat) order.
constexpr uint32_t kSupCap = 4608;      // the longest super-tile list sorted in LDS (46 KB per workgroup)
constexpr uint32_t kSupBuckets = 2048;  // the most buckets of a list sorted in LDS
constexpr uint32_t kSupItems = (kSupCap + kThreads - 1) / kThreads;
constexpr uint32_t kCover = 28;         // the cover bits' place in an entry's low word
constexpr uint32_t kCoarse = 256;       // a long list's chunking buckets
constexpr uint32_t kPass = 8;           // a long list's entries per thread per load batch
constexpr uint64_t kSortBits = ~(uint64_t(0xFu) << kCover);  // an entry's (depth bits, splat)
static_assert(kSupBuckets % kThreads == 0 && kSupBuckets <= kMaxBuckets, "super-tile bucket counts");

struct SuperShared {
  union {
    SortShared sh;  // the radix sort's counts
    struct {
      uint32_t start[kSupBuckets + 1];  // bucket counts, then their exclusive scan; start[nb] = m
      uint64_t entry[kSupCap];          // the entries grouped by bucket, then in sorted order
      uint32_t wmin[kWaves], wmax[kWaves], wsum[kWaves];
    } bkt;
  } u;
  uint32_t wtot[2][kWaves][4];  // the filter's per-wave counts per tile, double-buffered
  uint32_t cstart[kCoarse + 1];  // a long list's coarse buckets: counts, then starts
  uint32_t crun[kCoarse];        // their next free slots
  uint32_t chunk[kCoarse + 1];   // the first bucket of each chunk
  uint32_t nchunk;
};

#define GSR_SUPER_ORDER_PARAMS                                                                                    \
  uint64_t *__restrict__ list, const uint32_t *__restrict__ sup_start, const uint32_t *__restrict__ sup_total,       \
      uint32_t tiles_x, uint32_t tiles_y, const uint32_t *__restrict__ ranges, uint64_t pairs_cap,                 \
      const uint64_t *__restrict__ pairs_dev, const float *__restrict__ depths, uint32_t n,                         \
      uint32_t *__restrict__ vals_out, uint64_t *__restrict__ keys_out, uint32_t *gk0, uint32_t *gk1, uint32_t *gp0, \
      uint32_t *gp1

// Three workgroups per compute unit (LDS 49 KB each): six waves per SIMD, 80 registers.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void k_super_order(
    GSR_SUPER_ORDER_PARAMS) {
  __shared__ SuperShared ts;
  const uint64_t P = count_within(pairs_dev, pairs_cap);  // 0 when the pairs did not fit: nothing is written
  const uint32_t sup = blockIdx.x, sup_x = (tiles_x + 1) / 2;
  const uint32_t st = uint32_t(min<uint64_t>(sup_start[sup], P));
  const uint32_t m = uint32_t(min<uint64_t>(sup_total[sup], P - st));
  if (m == 0) return;
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint32_t bx = (sup % sup_x) * 2, by = (sup / sup_x) * 2;
  uint32_t tile[4], base[4];  // the four tiles and their lists' starts (uniform: held in scalar registers)
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t tx = bx + (j & 1u), ty = by + (j >> 1);
    tile[j] = tx < tiles_x && ty < tiles_y ? ty * tiles_x + tx : 0u;
    base[j] = __builtin_amdgcn_readfirstlane(tx < tiles_x && ty < tiles_y ? ranges[2 * tile[j]] : 0u);
  }
  const uint64_t* const lst = list + st;
  auto splat_at = [&](uint32_t e) -> uint32_t { return uint32_t(lst[e]) & ((1u << kCover) - 1u); };
  auto depth_bits = [&](uint32_t splat) -> uint32_t { return splat < n ? __float_as_uint(depths[splat]) : 0u; };

  // The extremes of kSupItems entries per thread (x[i] valid for tid + i kThreads < mc), over the workgroup.
  auto extremes = [&](const uint64_t* x, uint32_t mc, uint32_t& lo, uint32_t& hi) {
    uint32_t kmin = ~0u, kmax = 0;
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i)
      if (tid + i * kThreads < mc) kmin = min(kmin, uint32_t(x[i] >> 32)), kmax = max(kmax, uint32_t(x[i] >> 32));
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) ts.u.bkt.wmin[w] = kmin, ts.u.bkt.wmax[w] = kmax;
    __syncthreads();
    lo = ts.u.bkt.wmin[0], hi = ts.u.bkt.wmax[0];
#pragma unroll
    for (uint32_t q = 1; q < kWaves; ++q) lo = min(lo, ts.u.bkt.wmin[q]), hi = max(hi, ts.u.bkt.wmax[q]);
  };

  // Sorts mc <= kSupCap entries load(e) into ts.u.bkt.entry[0..mc) by (depth bits, splat). Buckets linear in the
  // depth value between the entries' extremes (monotone: fp32 subtraction, scaling by a positive factor and
  // truncation all preserve order), which spreads the workloads' uniform depths evenly (the per-tile order's map,
  // linear in the bits, crowds the top of a wide range: 35 against 33 us at 410k splats); each entry's rank among
  // the (depth bits, splat) of its bucket, then the entries moved to their ranks. Returns false, having sorted
  // nothing, when a bucket holds more than kBucketLimit entries (many equal depths), unless `force`.
  auto sort_in_lds = [&](uint32_t mc, auto load, bool force) -> bool {
    uint64_t x[kSupItems];
    uint32_t slot[kSupItems];
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i) {  // every load in flight at once (positions past mc read entry 0)
      const uint32_t e = tid + i * kThreads;
      x[i] = load(e < mc ? e : 0u);
    }
    const uint32_t half = (mc + 1) / 2;
    const uint32_t nb = min(kSupBuckets, max(kMinBuckets, half > 1 ? 1u << (32 - __clz(int(half - 1))) : 1u));
    for (uint32_t j = tid; j <= nb; j += kThreads) ts.u.bkt.start[j] = 0;
    uint32_t lo, hi;
    extremes(x, mc, lo, hi);
    const float lov = __uint_as_float(lo);
    const float scale = float(nb) / fmaxf(__uint_as_float(hi) - lov, 1e-30f);
    auto bucket = [&](uint32_t key) { return min(nb - 1, uint32_t((__uint_as_float(key) - lov) * scale)); };
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i)
      if (tid + i * kThreads < mc) slot[i] = atomicAdd(&ts.u.bkt.start[bucket(uint32_t(x[i] >> 32))], 1u);
    __syncthreads();
    const uint32_t biggest = scan_buckets(ts.u.bkt.start, nb, mc, ts.u.bkt.wsum);
    const bool crowded = __syncthreads_or(biggest > kBucketLimit);
    if (crowded && !force) return false;
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i)
      if (tid + i * kThreads < mc) ts.u.bkt.entry[ts.u.bkt.start[bucket(uint32_t(x[i] >> 32))] + slot[i]] = x[i];
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i) {
      const uint32_t q = tid + i * kThreads;
      slot[i] = ~0u;
      if (q < mc) {
        x[i] = ts.u.bkt.entry[q];
        const uint64_t me = x[i] & kSortBits;
        const uint32_t b = bucket(uint32_t(me >> 32));
        const uint32_t b0 = ts.u.bkt.start[b], b1 = ts.u.bkt.start[b + 1];
        uint32_t r = b0;
        for (uint32_t f = b0; f < b1; ++f) r += (ts.u.bkt.entry[f] & kSortBits) < me ? 1u : 0u;
        slot[i] = r;
      }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < kSupItems; ++i)
      if (slot[i] != ~0u) ts.u.bkt.entry[slot[i]] = x[i];
    __syncthreads();
    return true;
  };

  // The stable filter: the e-th of mc sorted entries entry_at(e) goes to the tiles its cover bits name, after the
  // `carry` entries of each tile that earlier calls wrote. Steps of kThreads consecutive entries, one per thread:
  // per tile, a ballot gives each entry its place among its wave's entries of that tile, the per-wave totals
  // (double-buffered in LDS, one barrier per step) its wave's place, so the entries of a tile leave each wave as one
  // contiguous run of stores.
  uint32_t carry[4] = {0u, 0u, 0u, 0u};
  auto filter = [&](uint32_t mc, auto entry_at) {
    for (uint32_t c0 = 0, step = 0; c0 < mc; c0 += kThreads, step ^= 1u) {
      const uint32_t e = c0 + tid;
      const uint64_t x = e < mc ? entry_at(e) : 0;
      const uint32_t spl = uint32_t(x) & ((1u << kCover) - 1u), key = uint32_t(x >> 32), mk = uint32_t(x) >> kCover;
      uint32_t below[4];
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        const uint64_t bal = __builtin_amdgcn_ballot_w64((mk >> j) & 1u);
        below[j] = uint32_t(__popcll(bal & lanemask_lt(lane)));
        if (lane == 0) ts.wtot[step][w][j] = uint32_t(__popcll(bal));
      }
      __syncthreads();
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (uint32_t q = 0; q < kWaves; ++q) {
          const uint32_t c = ts.wtot[step][q][j];
          before += q < w ? c : 0u;
          all += c;
        }
        // plain stores: a wave's run shares cache lines with the neighbouring waves' runs, which L2 merges
        // (non-temporal stores of these partial lines measured 43 against 35 us at 410k splats)
        if ((mk >> j) & 1u) {
          const uint64_t o = uint64_t(base[j]) + carry[j] + before + below[j];
          if (o < P) {  // always, when the tiles' totals and the cover bits agree; keeps a stray write in bounds
            vals_out[o] = spl;
            if (keys_out) keys_out[o] = (uint64_t(tile[j]) << 32) | key;
          }
        }
        carry[j] = __builtin_amdgcn_readfirstlane(carry[j] + all);
      }
    }
  };

  if (m <= kSupCap) {
    if (sort_in_lds(m, [&](uint32_t e) { return lst[e]; }, false)) {
      filter(m, [&](uint32_t e) { return ts.u.bkt.entry[e]; });
      return;
    }
  } else {
    // A longer list in chunks that LDS holds: kCoarse buckets linear in the depth value between the list's
    // extremes (equal depths share one) count the entries and partition them into the arena (low words in gk0,
    // high words in gk1, at the list's stretch); runs of consecutive buckets of at most kSupCap entries are then
    // sorted and filtered one after the other (the filter carries each tile's count from chunk to chunk). A bucket
    // of more than kSupCap entries sends the list to the radix sort instead (decided before anything is written); a
    // chunk with a crowded bucket is sorted by the radix sort on its own.
    // f(e, entry) for every entry, kPass loads per thread in flight at once
    auto each_entry = [&](auto f) {
      for (uint32_t e0 = 0; e0 < m; e0 += kPass * kThreads) {
        uint64_t x[kPass];
#pragma unroll
        for (uint32_t i = 0; i < kPass; ++i) {
          const uint32_t e = e0 + i * kThreads + tid;
          x[i] = lst[e < m ? e : 0u];
        }
#pragma unroll
        for (uint32_t i = 0; i < kPass; ++i)
          if (e0 + i * kThreads + tid < m) f(e0 + i * kThreads + tid, x[i]);
      }
    };
    uint32_t kmin = ~0u, kmax = 0;
    each_entry([&](uint32_t, uint64_t x) {
      const uint32_t k = uint32_t(x >> 32);
      kmin = min(kmin, k), kmax = max(kmax, k);
    });
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) ts.u.bkt.wmin[w] = kmin, ts.u.bkt.wmax[w] = kmax;
    for (uint32_t c = tid; c <= kCoarse; c += kThreads) ts.cstart[c] = 0;
    __syncthreads();
    uint32_t lo = ts.u.bkt.wmin[0], hi = ts.u.bkt.wmax[0];
#pragma unroll
    for (uint32_t q = 1; q < kWaves; ++q) lo = min(lo, ts.u.bkt.wmin[q]), hi = max(hi, ts.u.bkt.wmax[q]);
    const float lov = __uint_as_float(lo);
    const float cscale = float(kCoarse) / fmaxf(__uint_as_float(hi) - lov, 1e-30f);
    auto coarse = [&](uint32_t key) { return min(kCoarse - 1, uint32_t((__uint_as_float(key) - lov) * cscale)); };
    each_entry([&](uint32_t, uint64_t x) { atomicAdd(&ts.cstart[coarse(uint32_t(x >> 32))], 1u); });
    __syncthreads();
    const uint32_t cnt = tid < kCoarse ? ts.cstart[tid] : 0u;
    if (!__syncthreads_or(cnt > kSupCap)) {
      const uint32_t first = block_exclusive_scan<uint32_t, kThreads>(cnt, nullptr, ts.u.bkt.wsum);
      if (tid < kCoarse) ts.cstart[tid] = first, ts.crun[tid] = first;
      if (tid == 0) ts.cstart[kCoarse] = m;
      __syncthreads();
      if (tid == 0) {  // chunk boundaries: runs of consecutive buckets of at most kSupCap entries
        uint32_t nch = 0, acc = 0;
        ts.chunk[0] = 0;
        for (uint32_t c = 0; c < kCoarse; ++c) {
          const uint32_t k = ts.cstart[c + 1] - ts.cstart[c];
          if (acc + k > kSupCap) ts.chunk[++nch] = c, acc = 0;
          acc += k;
        }
        ts.chunk[++nch] = kCoarse;
        ts.nchunk = nch;
      }
      each_entry([&](uint32_t, uint64_t x) {
        const uint32_t q = atomicAdd(&ts.crun[coarse(uint32_t(x >> 32))], 1u);
        gk0[st + q] = uint32_t(x);
        gk1[st + q] = uint32_t(x >> 32);
      });
      __syncthreads();  // the partition's global writes are seen by the whole workgroup after the barrier
      const uint32_t nch = ts.nchunk;
      for (uint32_t k = 0; k < nch; ++k) {
        const uint32_t e0 = ts.cstart[ts.chunk[k]], mc = ts.cstart[ts.chunk[k + 1]] - e0;
        if (mc == 0) continue;  // not reached: every chunk holds an entry (uniform)
        const uint32_t* const lw = gk0 + st + e0;
        const uint32_t* const hw = gk1 + st + e0;
        if (sort_in_lds(mc, [&](uint32_t e) { return (uint64_t(hw[e]) << 32) | lw[e]; }, false)) {
          filter(mc, [&](uint32_t e) { return ts.u.bkt.entry[e]; });
        } else {
          // a crowded chunk (many equal or nearly equal depths): the radix sort through the arena, keys in gp0 and
          // gp1 and positions in the list's own stretch, free once partitioned (its 64-bit words as 2m 32-bit ones)
          uint32_t* const free32 = reinterpret_cast<uint32_t*>(list + st);
          uint32_t *k0 = gp0 + st + e0, *k1 = gp1 + st + e0, *p0 = free32 + e0, *p1 = free32 + m + e0;
          auto chunk_splat = [&](uint32_t e) -> uint32_t { return lw[e] & ((1u << kCover) - 1u); };
          const uint32_t res = radix_order(k0, k1, p0, p1, mc, false, chunk_splat, depth_bits, ts.u.sh);
          const uint32_t* const kr = res ? k1 : k0;
          const uint32_t* const pr = res ? p1 : p0;
          filter(mc, [&](uint32_t e) { return (uint64_t(kr[e]) << 32) | lw[pr[e]]; });
        }
        __syncthreads();  // the next chunk reuses the LDS
      }
      return;
    }
  }
  // otherwise the radix sort through the arena (a barrier above ends every read of the LDS)
  uint32_t *k0 = gk0 + st, *k1 = gk1 + st, *p0 = gp0 + st, *p1 = gp1 + st;
  const uint32_t res = radix_order(k0, k1, p0, p1, m, false, splat_at, depth_bits, ts.u.sh);
  const uint32_t* kr = res ? k1 : k0;
  const uint32_t* pr = res ? p1 : p0;
  filter(m, [&](uint32_t e) { return (uint64_t(kr[e]) << 32) | uint32_t(lst[pr[e]]); });
}

}  // namespace

void launch_tile_depth(hipStream_t s, const uint32_t* list, const uint32_t* list_vals, uint32_t idx_bits,
                       bool ordered, const uint32_t* ranges, uint64_t pairs_cap, const uint64_t* pairs_dev,
                       uint32_t num_tiles, const float* depths, uint32_t n, uint32_t* vals_out, uint64_t* keys_out,
                       uint64_t* gent, uint32_t* gk0, uint32_t* gk1, uint32_t* gp0, uint32_t* gp1) {
  if (num_tiles <= kMaxGrid) {
    if (num_tiles)
      hipLaunchKernelGGL(k_tile_depth<false>, dim3(num_tiles), dim3(kThreads), 0, s, list, list_vals, idx_bits,
                         ordered, ranges, pairs_cap, pairs_dev, num_tiles, depths, n, vals_out, keys_out, gent, gk0,
                         gk1, gp0, gp1);
  } else {
    hipLaunchKernelGGL(k_tile_depth<true>, dim3(kMaxGrid), dim3(kThreads), 0, s, list, list_vals, idx_bits, ordered,
                       ranges, pairs_cap, pairs_dev, num_tiles, depths, n, vals_out, keys_out, gent, gk0, gk1, gp0,
                       gp1);
  }
}

uint32_t tile_depth_capacity() { return kCap; }

void launch_super_order(hipStream_t s, uint64_t* list, const uint32_t* sup_start, const uint32_t* sup_total,
                        uint32_t num_sup, uint32_t tiles_x, uint32_t tiles_y, const uint32_t* ranges,
                        uint64_t pairs_cap, const uint64_t* pairs_dev, const float* depths, uint32_t n,
                        uint32_t* vals_out, uint64_t* keys_out, uint32_t* gk0, uint32_t* gk1, uint32_t* gp0,
                        uint32_t* gp1) {
  if (num_sup)
    hipLaunchKernelGGL(k_super_order, dim3(num_sup), dim3(kThreads), 0, s, list, sup_start, sup_total, tiles_x,
                       tiles_y, ranges, pairs_cap, pairs_dev, depths, n, vals_out, keys_out, gk0, gk1, gp0, gp1);
}

}  // namespace gsr
