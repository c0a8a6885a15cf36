// Backward rasterization: one 256-thread workgroup per 16x16 tile (four wave64, one 8x8 block each), one pixel per
// thread, same LDS staging and per-wave cull as the forward. Each lane replays its forward decisions (the shared
// evaluate()) up to its last contributor and forms the 9 gradient terms of each splat it composited; a wave stops
// at the largest last contributor among its lanes. Per splat and wave:
//   - if no lane of the wave composited it, nothing is reduced or added (W1 warp sparse skip + exp-skip page,
//     section 1 row "W1a": an all-invalid wave would only add +0.0);
//   - otherwise the 9 terms are summed over the wave by a transposing butterfly (permlane32/16 swaps, then DPP) that
//     leaves each total in one lane, and those nine lanes add them into the workgroup's LDS accumulator of that
//     splat;
// after each batch one thread per splat adds the accumulated 9 values to splats_grad with global float atomics,
// which complete while the next batch is processed (the loop's barriers order LDS only).
// The per-pixel terms follow the forward-order form after = C_final - acc - mine of the M3 per-splat backward page
// (section 1, rows "brush's actual structure" and "differences").
#include <type_traits>

#include "gsr_internal.hpp"
#include "raster_common.hpp"

namespace gsr {
namespace {

constexpr uint32_t kGrads = 9;

// v + (v of the lane selected by kCtrl). Every control used here selects a lane of the same 16-lane row and all 64
// lanes are active, so bound_ctrl (read 0 from an invalid lane) never applies; setting it lets the compiler fold the
// move into a single v_add_f32_dpp.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true);
  return v + __int_as_float(moved);
}

__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}

__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_get(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Sums each of the 9 values in d over the 64 lanes of the wave with a transposing butterfly: at every halving step
// a lane keeps one value of each pair and adds its partner's copy of it, so the number of values per lane halves
// while the lane set summed doubles. Steps: the two 32-lane halves (v_permlane32_swap: one swap exchanges a half of
// each of two registers, and adding the pair gives each half the sum of one of them), the row pairs of each half
// (v_permlane16_swap, likewise), lanes i and i^8 of a row (DPP row_ror:8 with selects), lanes i and 7-i of a half
// row (DPP row_half_mirror with selects), then lanes i^2 and i^1 (DPP quad permutes, plain sums). Every lane ends
// with the 64-lane total of one value; which one depends only on the lane's position (see transpose_index).
// 29 VALU instructions instead of 36 DPP adds for row sums plus a cross-row step for all 9 values.
__device__ __forceinline__ float transpose_reduce(const float (&d)[9], uint32_t lane) {
  float r[5];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float a = d[2 * m], b = d[2 * m + 1];
    swap32(a, b);
    r[m] = a + b;
  }
  {
    float a = d[8], b = 0.0f;
    swap32(a, b);
    r[4] = a + b;
  }
  float s[3];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    float a = r[2 * n], b = r[2 * n + 1];
    swap16(a, b);
    s[n] = a + b;
  }
  {
    float a = r[4], b = 0.0f;
    swap16(a, b);
    s[2] = a + b;
  }
  const bool lo8 = (lane & 8u) == 0;
  const float t0 = (lo8 ? s[0] : s[1]) + dpp_get<0x128>(lo8 ? s[1] : s[0]);  // row_ror:8 pairs i with i ^ 8
  const float t1 = (lo8 ? s[2] : 0.0f) + dpp_get<0x128>(lo8 ? 0.0f : s[2]);
  const bool lo4 = (lane & 4u) == 0;
  float u = (lo4 ? t0 : t1) + dpp_get<0x141>(lo4 ? t1 : t0);  // row_half_mirror pairs i with 7 - i
  u = dpp_add<0x4E>(u);                                        // quad_perm [2,3,0,1]
  u = dpp_add<0xB1>(u);                                        // quad_perm [1,0,3,2]
  return u;
}

// Which of the 9 values transpose_reduce leaves in this lane (-1: a padding slot), found by running the same
// network on the indices 1..9, identical in every lane: the total is 64 (index + 1). Must be called with all 64
// lanes active (the network reads other lanes). The inputs carry a lane-dependent +0 so that the compiler keeps
// the lane exchanges instead of folding them as uniform constants.
__device__ __forceinline__ int transpose_index(uint32_t lane) {
  const float zero = 0.0f * float(lane);
  float idx[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) idx[q] = float(q + 1) + zero;
  const float t = transpose_reduce(idx, lane);
  return int(t * (1.0f / 64.0f) + 0.5f) - 1;
}

// Zeroes count floats, four per thread: one 16-byte store when p is 16-byte aligned and all four exist.
__global__ __launch_bounds__(kTilePixels) void k_zero(float* __restrict__ p, uint64_t count, bool aligned) {
  const uint64_t i = (uint64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (aligned && i + 4 <= count) {
    *reinterpret_cast<float4*>(p + i) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else {
#pragma unroll
    for (uint64_t q = 0; q < 4; ++q)
      if (i + q < count) p[i + q] = 0.0f;
  }
}

// kSkip: each wave walks only the staged splats that can reach alpha >= 1/255 in its 8x8 block, and skips the
// reduction of a splat no lane composited. Both skip only additions of +0.0 and certain rejects.
// kDet: sums that do not depend on scheduling. Waves 0-1 and waves 2-3 each add into an accumulator of their own:
// float addition is commutative, so two additions to a zeroed cell give the same bits in either order (three would
// not); the two accumulators are added at the flush. Each tile's totals are added into 128-bit fixed-point sums
// (value x 2^48, rounded to nearest) with two 64-bit integer atomics: integer addition is exact, so any order of the
// tiles gives the same bits. The low word starts at 2^63 (a bias taken off at the end), so the high word is touched
// only when a running sum passes +-32768. Tile totals that are not finite, or of magnitude 2^79 and up, set bits in
// a per-splat flag word instead (NaN; +inf; -inf), from which the conversion rebuilds what a float sum would give.
constexpr double kFixedScale = 0x1p48;
constexpr unsigned long long kFixedBias = 0x8000000000000000ull;

struct FixedSums {
  unsigned long long* words;  // [n * 9][2]: low word (biased), high word
  uint32_t* flags;            // [n]: bit q NaN, bit 9 + q +inf, bit 18 + q -inf, for value q
};

__device__ __forceinline__ void add_fixed(FixedSums acc, uint32_t idx, uint32_t q, float g) {
  const double t = double(g) * kFixedScale;  // exact
  if (!(fabs(t) < 0x1p127)) {
    const uint32_t bit = g != g ? q : (g > 0.0f ? kGrads + q : 2 * kGrads + q);
    atomicOr(acc.flags + idx, 1u << bit);
    return;
  }
  __int128 v;
  if (fabs(t) < 0x1p62) {
    v = __double2ll_rn(t);
  } else {  // an integer m 2^(e - 53) with |m| < 2^53 and e - 53 in [10, 74]
    int e;
    const double f = frexp(t, &e);
    v = static_cast<__int128>(static_cast<long long>(f * 0x1p53)) << (e - 53);
  }
  const unsigned long long lo = static_cast<unsigned long long>(v);
  const long long hi = static_cast<long long>(v >> 64);
  unsigned long long* word = acc.words + 2 * (size_t(idx) * kGrads + q);
  const unsigned long long old = atomicAdd(word, lo);
  const long long carry_hi = hi + (old + lo < old ? 1 : 0);  // the low word wrapped: carry into the high word
  if (carry_hi != 0) atomicAdd(word + 1, static_cast<unsigned long long>(carry_hi));
}

__global__ __launch_bounds__(kTilePixels) void k_fixed_clear(FixedSums acc, uint64_t count, uint32_t n) {
  const uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) {
    acc.words[2 * i] = kFixedBias;
    acc.words[2 * i + 1] = 0;
  }
  if (i < n) acc.flags[i] = 0;
}

__global__ __launch_bounds__(kTilePixels) void k_fixed_to_float(FixedSums acc, float* __restrict__ out,
                                                                uint64_t count) {
  const uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const uint32_t idx = uint32_t(i / kGrads), q = uint32_t(i - uint64_t(idx) * kGrads);
  const uint32_t fl = acc.flags[idx];
  const bool nan = (fl >> q) & 1u, pinf = (fl >> (kGrads + q)) & 1u, ninf = (fl >> (2 * kGrads + q)) & 1u;
  float r;
  if (nan || (pinf && ninf)) {
    r = __builtin_nanf("");
  } else if (pinf || ninf) {
    r = pinf ? __builtin_inff() : -__builtin_inff();
  } else {
    const long long lo = static_cast<long long>(acc.words[2 * i] ^ kFixedBias);  // the sum is hi 2^64 + lo
    const long long hi = static_cast<long long>(acc.words[2 * i + 1]);
    if (hi == 0)
      r = static_cast<float>(lo) * float(1.0 / kFixedScale);  // one rounding; the scaling is exact
    else
      r = float((double(hi) * 0x1p64 + double(lo)) * (1.0 / kFixedScale));
  }
  out[i] = r;
}

#define GSR_BACKWARD_PARAMS                                                                                        \
  const float *__restrict__ splats, uint32_t n, const uint32_t *__restrict__ vals,                                  \
      const uint32_t *__restrict__ ranges, uint32_t num_pairs, uint32_t tiles_x, uint32_t width, uint32_t height,   \
      const float4 *__restrict__ out_rgba, const uint32_t *__restrict__ last_contrib,                               \
      const float4 *__restrict__ v_out, float *__restrict__ splats_grad, FixedSums fixed,                           \
      const uint32_t *__restrict__ tile_order, uint32_t num_tiles
#define GSR_BACKWARD_ARGS \
  splats, n, vals, ranges, num_pairs, tiles_x, width, height, out_rgba, last_contrib, v_out, splats_grad, fixed, \
      tile_order, num_tiles

// The nine per-splat sums of a wave, as moments. With (u, t) = pixel centre - tile centre (exact: multiples of 0.5
// in [-7.5, 7.5]) and per lane v = dL/do = dL/dalpha G (0 where the lane did not composite or alpha is clamped) and
// w = alpha T (0 where it did not composite), the sums taken are
//   S0..S5 = sum v (1, u, t, u^2, u t, t^2),   C0..C2 = sum w (g_r, g_g, g_b),
// accumulated per staged splat in LDS as [S0..S5, C0..C2] over the tile's four waves. At the batch's end the splat's
// mean and conic gradients follow from them with xl = x - tile centre x, yl = y - tile centre y (dx = u - xl,
// dy = t - yl): sum v dx = S1 - xl S0, sum v dx^2 = S3 - xl (S1 + sum v dx), and likewise; these are the sums of
// v dx, v dy, v dx^2, v dx dy, v dy^2 the gradient is made of, each with the rounding of a plain fp32 sum of terms
// of the same size. The moments are a contraction over the wave's 64 pixels of two per-lane values against fixed
// per-pixel features (a dense 9 x 64 by 64 x 2 product per splat), which the matrix cores take: each compositing
// splat's v and w go to a per-wave LDS buffer of columns, and every kChunk splats one chain of 16
// v_mfma_f32_16x16x4f32 contracts them. Waves that fall back to the lane butterfly (non-finite upstream gradients,
// the deterministic option, the skip-free A/B form) reduce the same nine values.
constexpr uint32_t kBatch = 96;       // splats staged per batch (a wave and a half stage them): with the column
                                      // buffers the workgroup's LDS stays under 26.6 KB, six per compute unit
constexpr uint32_t kChunk = 8;        // splats per MFMA contraction
constexpr uint32_t kColStride = 68;   // floats per buffer column: 64 pixels + 4, so the 16 columns' reads of one
                                      // 16-byte group fall on 16 distinct groups of banks
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Moments and colour sums of a staged splat -> its nine gradient values in record order (x, y, a, b, c, r, g, b, o):
// dL/dmean = o (a Sx + b Sy, b Sx + c Sy) = 2 o (ha Sx + hb Sy, hb Sx + hc Sy), dL/d(a, b, c) = -o (Sxx / 2, Sxy,
// Syy / 2), dL/d rgb = C, dL/do = S0.
__device__ __forceinline__ void moments_to_grads(float* acc, const StagedSplat& sp, float tcx, float tcy) {
  const float S0 = acc[0], S1 = acc[1], S2 = acc[2], S3 = acc[3], S4 = acc[4], S5 = acc[5];
  const float c0 = acc[6], c1 = acc[7], c2 = acc[8];
  float g0 = 0.0f, g1 = 0.0f, g2 = 0.0f, g3 = 0.0f, g4 = 0.0f;
  if (S0 != 0.0f || S1 != 0.0f || S2 != 0.0f || S3 != 0.0f || S4 != 0.0f || S5 != 0.0f) {
    const float xl = sp.x - tcx, yl = sp.y - tcy;
    const float Sx = S1 - xl * S0;
    const float Sy = S2 - yl * S0;
    const float Sxx = S3 - xl * (S1 + Sx);
    const float Sxy = (S4 - xl * S2) - yl * Sx;
    const float Syy = S5 - yl * (S2 + Sy);
    const float o2 = sp.o + sp.o;
    g0 = o2 * __fmaf_rn(sp.ha, Sx, sp.hb * Sy);
    g1 = o2 * __fmaf_rn(sp.hb, Sx, sp.hc * Sy);
    g2 = (-0.5f * sp.o) * Sxx;
    g3 = -sp.o * Sxy;
    g4 = (-0.5f * sp.o) * Syy;
  }
  acc[0] = g0, acc[1] = g1, acc[2] = g2, acc[3] = g3, acc[4] = g4;
  acc[5] = c0, acc[6] = c1, acc[7] = c2, acc[8] = S0;
}

template <bool kSkip, bool kDet>
__device__ __forceinline__ void backward_tile(GSR_BACKWARD_PARAMS) {
  constexpr uint32_t kWaves = kTilePixels / kWave;
  constexpr uint32_t kStageWaves = (kBatch + kWave - 1) / kWave;  // waves whose lanes stage a splat
  constexpr bool kMfmaForm = kSkip && !kDet;  // the matrix-core reduction (the default configuration)
  __shared__ StagedSplat s_sp[kBatch];
  __shared__ double s_exp2[64];  // 2^(j/32) table of the exact exponential
  constexpr uint32_t kAcc = kDet ? 2 : 1;  // accumulators: one per pair of waves, or one for all four
  __shared__ float s_acc[kAcc][kBatch][kGrads];
  __shared__ uint64_t s_mask[kWaves][kStageWaves];  // [reading wave][staging wave]
  __shared__ __align__(16) float s_cols[kMfmaForm ? kWaves : 1][kMfmaForm ? 2 * kChunk : 1][kColStride];
  __shared__ uint32_t s_max_last;
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int slot_any = transpose_index(lane);               // all lanes take part in the exchanges
  const int my_slot = (lane & 3u) == 0 ? slot_any : -1;      // the term this lane totals (4 copies; one adds)
  const uint32_t tile = tile_order[blockIdx.x];  // slowest expected first (a permutation of the tiles)
  if (tile >= num_tiles) return;                 // not reachable with a permutation; keeps reads in bounds
  load_exp_table(s_exp2);                        // the barriers below order it
  const uint32_t tx0 = (tile % tiles_x) * kTile, ty0 = (tile / tiles_x) * kTile;
  const uint32_t px = tx0 + lane_px(w, lane), py = ty0 + lane_py(w, lane);
  const bool inside = px < width && py < height;
  const uint32_t start = min(ranges[2 * tile], num_pairs);
  const uint32_t end = max(start, min(ranges[2 * tile + 1], num_pairs));
  const float cx = float(px) + 0.5f, cy = float(py) + 0.5f;
  const float tcx = float(tx0) + 8.0f, tcy = float(ty0) + 8.0f;  // the tile's centre, origin of the moments
  const float mu = cx - tcx, mt = cy - tcy;                        // exact
  const float muu = mu * mu, mut = mu * mt, mtt = mt * mt;         // exact

  uint32_t last = 0;
  float Cr = 0.0f, Cg = 0.0f, Cb = 0.0f, gr = 0.0f, gg = 0.0f, gb = 0.0f;
  if (inside) {
    const size_t p = size_t(py) * width + px;
    last = min(last_contrib[p], end - start);
    const float4 c = out_rgba[p];
    const float4 g = v_out[p];
    Cr = c.x;
    Cg = c.y;
    Cb = c.z;
    gr = g.x;
    gg = g.y;
    gb = g.z;
  }
  // A lane that does not composite a splat has wgt = 0, so its colour terms wgt g are exact zeros unless its
  // upstream gradient g is not finite; waves holding such a pixel select the zeros explicitly (lane butterfly).
  const bool g_finite = __builtin_isfinite(gr) && __builtin_isfinite(gg) && __builtin_isfinite(gb);
  const bool wave_g_finite = __builtin_amdgcn_readfirstlane(uint32_t(__ballot(!g_finite) == 0)) != 0;
  if (tid == 0) s_max_last = 0;
  for (uint32_t i = tid; i < kAcc * kBatch * kGrads; i += kTilePixels) (&s_acc[0][0][0])[i] = 0.0f;
  // the wave's bound: the largest last contributor among its lanes
  uint32_t wave_last = last;
  for (uint32_t off = 32; off > 0; off >>= 1) wave_last = max(wave_last, uint32_t(__shfl_xor(int(wave_last), off)));
  wave_last = __builtin_amdgcn_readfirstlane(wave_last);
  // Matrix operand A of the contraction, one register per instruction i = 0..15 of a chain: lane l holds feature
  // m = l mod 16 of the wave's pixel q = 4 i + l / 16 (1, u, t, u^2, u t, t^2, g_r, g_g, g_b, then zeros). Rows 6..8
  // multiply the v columns and rows 0..5 the w columns into sums nobody reads.
  float amat[16];
  if constexpr (kMfmaForm) {
    const uint32_t m = lane & 15u;
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {
      const uint32_t q = 4 * i + (lane >> 4);
      const float qu = float(lane_px(w, q)) + 0.5f - 8.0f, qt = float(lane_py(w, q)) + 0.5f - 8.0f;
      const float qg0 = __shfl(gr, int(q)), qg1 = __shfl(gg, int(q)), qg2 = __shfl(gb, int(q));
      float f = 0.0f;
      f = m == 0 ? 1.0f : f;
      f = m == 1 ? qu : f;
      f = m == 2 ? qt : f;
      f = m == 3 ? qu * qu : f;
      f = m == 4 ? qu * qt : f;
      f = m == 5 ? qt * qt : f;
      f = m == 6 ? qg0 : f;
      f = m == 7 ? qg1 : f;
      f = m == 8 ? qg2 : f;
      amat[i] = f;
    }
  }
  __syncthreads();
  if (lane == 0) atomicMax(&s_max_last, wave_last);
  __syncthreads();
  const uint32_t stop = start + s_max_last;

  // The batch loop, instantiated twice: kGuard selects the colour terms' explicit zeros (waves with a non-finite
  // upstream gradient), reduced by the lane butterfly. Waves of one workgroup may run different instantiations;
  // both pass the same barriers and fill the accumulator with the same nine values.
  auto batches = [&](auto guard) {
  constexpr bool kGuard = decltype(guard)::value;
  constexpr bool kMfma = kMfmaForm && !kGuard;
  float T = 1.0f, ar = 0.0f, ag = 0.0f, ab = 0.0f;
  // this lane's pixel's place in a column: instruction i = q / 4 reads k-slot q mod 4 (lanes 16 (q mod 4) ...)
  float* const col_base = &s_cols[kMfma ? w : 0][0][0];
  float* const my_cell = col_base + (((lane & 3u) << 4) | (lane >> 2));
  uint32_t used = 0;  // splats in the current chunk (wave-uniform)
  int slot_j = 0;     // lane s holds the batch slot of the chunk's splat s
  // Contracts the chunk's `count` splats and adds their sums to the accumulator. All 64 lanes, uniform flow.
  auto contract = [&](uint32_t count) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    // B operands: column n = lane mod 16, k-slot lane / 16: floats 16 (lane / 16) + i of the column, i = 0..15
    const floatx4* src = reinterpret_cast<const floatx4*>(col_base + (lane & 15u) * kColStride + ((lane >> 4) << 4));
    const floatx4 b0 = src[0], b1 = src[1], b2 = src[2], b3 = src[3];
    floatx4 d = {0.0f, 0.0f, 0.0f, 0.0f};
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[0], b0[0], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[1], b0[1], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[2], b0[2], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[3], b0[3], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[4], b1[0], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[5], b1[1], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[6], b1[2], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[7], b1[3], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[8], b2[0], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[9], b2[1], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[10], b2[2], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[11], b2[3], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[12], b3[0], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[13], b3[1], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[14], b3[2], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(amat[15], b3[3], d, 0, 0, 0);
    // lane l holds rows 4 (l / 16) + r of column l mod 16: column 2 s carries v (rows 0..5 useful), column 2 s + 1
    // carries w (rows 6..8 useful) of the chunk's splat s
    const uint32_t n = lane & 15u, sl = n >> 1, kind = n & 1u, row0 = (lane >> 4) << 2;
    const int jb = __shfl(slot_j, int(sl));
    if (sl < count) {
      float* acc = s_acc[0][jb];
#pragma unroll
      for (uint32_t r = 0; r < 4; ++r) {
        const uint32_t row = row0 + r;
        if (kind == 0 ? row < 6u : (row >= 6u && row < 9u)) atomicAdd(acc + row, d[r]);
      }
    }
    // the next chunk's stores go to the columns these reads came from (same wave: LDS keeps its order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  for (uint32_t b0 = start; b0 < stop; b0 += kBatch) {
    const uint32_t k = b0 + tid;
    uint32_t reach = 0;
    if (tid < kBatch && k < stop) {
      const StagedSplat st = stage_splat(splats, vals[k], n);
      s_sp[tid] = st;
      reach = kSkip ? reach_mask(st, float(tx0) + 0.5f, float(ty0) + 0.5f) : 0xFu;
    }
    if (w < kStageWaves) {
#pragma unroll
      for (uint32_t q = 0; q < kWaves; ++q) {
        const uint64_t bits = __ballot((reach >> q) & 1u);
        if (lane == 0) s_mask[q][w] = bits;
      }
    }
    lds_barrier();
    const uint32_t rel0 = b0 - start;
    for (uint32_t sw = 0; sw < kStageWaves; ++sw) {
      uint64_t m = uniform64(s_mask[w][sw]);
      while (m) {
        const uint32_t j = sw * kWave + uint32_t(__builtin_ctzll(m));
        m &= m - 1;
        if (rel0 + j >= wave_last) {
          m = 0;
          sw = kStageWaves;  // past every lane's last contributor: done with this batch and the tile
          break;
        }
        // the whole record in three 16-byte reads from one address register
        const float4* rec = reinterpret_cast<const float4*>(&s_sp[j]);
        const float4 q0 = rec[0], q1 = rec[1], q2 = rec[2];
        StagedSplat s;
        s.x = q0.x, s.y = q0.y, s.ha = q0.z, s.b = q0.w;
        s.hc = q1.x, s.o = q1.y, s.r = q1.z, s.g = q1.w;
        s.bl = q2.x, s.lr = q2.y, s.hb = q2.z, s.idx = __float_as_uint(q2.w);
        Eval e;  // dx and dy are set in every lane; G, oG and alpha only where the evaluation passed
        const bool contrib = evaluate<false>(s, cx, cy, e, s_exp2) & (rel0 + j < last);
        // Every lane forms the terms; in a lane that did not composite the splat, alpha = 0 and v = 0 make them
        // +-0 and leave T and acc as they are (the splat is binned, so its values are finite). A compositing lane
        // has alpha >= 1/255, so the skip tests alpha itself (one compare into the mask).
        const float alpha = contrib ? e.alpha : 0.0f;
        if (kSkip && __builtin_amdgcn_ballot_w64(alpha != 0.0f) == 0) continue;  // no lane composited this splat
        const float one_m = 1.0f - alpha;
        const float wgt = alpha * T;
        const float mr = s.r * wgt, mg = s.g * wgt, mb = s.bl * wgt;
        // dL/dalpha = T (g . rgb) - (g . after) / (1 - alpha), after = C_final - acc - mine, per channel as
        // (C_final - acc) - mine: after is a difference of nearly equal values that 1 / (1 - alpha) amplifies, so
        // its rounding follows that of the plain per-channel evaluation
        const float g_rgb = __fmaf_rn(gb, s.bl, __fmaf_rn(gg, s.g, gr * s.r));
        const float g_after = __fmaf_rn(gb, (Cb - ab) - mb, __fmaf_rn(gg, (Cg - ag) - mg, gr * ((Cr - ar) - mr)));
        const float dl_da = __fmaf_rn(T, g_rgb, -g_after * __builtin_amdgcn_rcpf(one_m));
        // alpha depends on o and sigma only below the clamp: the opacity and geometry terms get a 0 / 1 factor.
        // v = dL/do = dL/dalpha G; the geometry sums are moments of v (see moments_to_grads)
        const float v = (contrib && e.oG < kAlphaMax) ? dl_da * e.G : 0.0f;
        ar = ar + mr;
        ag = ag + mg;
        ab = ab + mb;
        T = T * one_m;
        if constexpr (kMfma) {
          // this lane's v and w into the chunk's columns 2 used and 2 used + 1
          my_cell[(2 * used) * kColStride] = v;
          my_cell[(2 * used + 1) * kColStride] = wgt;
          asm volatile("v_writelane_b32 %0, %1, m0" : "+v"(slot_j) : "s"(j), "{m0}"(used));
          if (++used == kChunk) {
            contract(kChunk);
            used = 0;
          }
        } else {
          float d[kGrads];
          d[0] = v;
          d[1] = v * mu;
          d[2] = v * mt;
          d[3] = v * muu;
          d[4] = v * mut;
          d[5] = v * mtt;
          d[6] = wgt * gr;
          d[7] = wgt * gg;
          d[8] = wgt * gb;
          if constexpr (kGuard) {
            d[6] = contrib ? d[6] : 0.0f;
            d[7] = contrib ? d[7] : 0.0f;
            d[8] = contrib ? d[8] : 0.0f;
          }
          // Wave totals of the 9 terms; nine lanes add them to the LDS accumulator (distinct addresses).
          const float x = transpose_reduce(d, lane);
          if (my_slot >= 0) atomicAdd(&s_acc[kDet ? w >> 1 : 0][j][my_slot], x);
        }
      }
    }
    if constexpr (kMfma) {
      if (used) {
        contract(used);
        used = 0;
      }
    }
    lds_barrier();
    // Per staged splat, its moments become its nine gradient values (moments_to_grads).
    const uint32_t staged = min(kBatch, stop - b0);
    if (tid < staged) {
      float* acc = s_acc[0][tid];
      if constexpr (kDet) {
#pragma unroll
        for (uint32_t q = 0; q < kGrads; ++q) acc[q] += s_acc[1][tid][q];
      }
      moments_to_grads(acc, s_sp[tid], tcx, tcy);
    }
    lds_barrier();
    // Flush: the batch's accumulator is read in its [slot][value] order, so the 64 lanes of an atomic instruction
    // add to the consecutive values of about seven splats (a few cache lines) rather than to 64 scattered records.
    for (uint32_t f = tid; f < staged * kGrads; f += kTilePixels) {
      const uint32_t slot = f / kGrads, q = f - slot * kGrads;
      const float g = (&s_acc[0][0][0])[f];
#pragma unroll
      for (uint32_t a = 0; a < kAcc; ++a) (&s_acc[a][0][0])[f] = 0.0f;
      const uint32_t idx = s_sp[slot].idx;
      if (idx != 0xFFFFFFFFu && (!kSkip || g != 0.0f)) {
        if constexpr (kDet)
          add_fixed(fixed, idx, q, g);
        else
          atomicAdd(splats_grad + size_t(idx) * kGrads + q, g);
      }
    }
    lds_barrier();
  }
  };
  if (wave_g_finite)
    batches(std::false_type{});
  else
    batches(std::true_type{});
}

// Per-splat backward (the loop order of the M3 per-splat backward page: a thread owns a splat and visits the
// tile's pixels in a diagonal schedule, so that its nine sums stay in the thread and need no cross-lane reduction).
// Here each wave owns one 8x8 block of the tile and needs no barrier after the set-up: it takes the tile's list up
// to the block's last contributor in chunks of 64, keeps the splats the block cull lets through (compacted in list
// order, lane j = the chunk's j-th such splat), and sweeps: at step t lane j evaluates pixel p = t - j of the
// block. The pixel's state before the splat (T and the accumulated colour) comes from lane j - 1, which held that
// pixel one step earlier (a one-lane shift of the wave), or for lane 0 from LDS, where the last lane of the
// previous chunk left it. Every (pixel, splat) term is the per-pixel kernel's; a lane adds its splat's terms in
// pixel order, applies the splat's factors once per chunk and adds the nine results to splats_grad (float atomics,
// or the fixed-point sums under kDet, which need no other care: each sum is formed in a fixed order).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kWaveShr1 = 0x138;  // DPP wave_shr:1, lane i takes lane i - 1

template <bool kSkip, bool kDet>
__device__ __forceinline__ void backward_splat_tile(GSR_BACKWARD_PARAMS) {
  constexpr uint32_t kWaves = kTilePixels / kWave;
  __shared__ double s_exp2[64];
  __shared__ float4 s_pix[kWaves][kWave];    // C_final rgb, last contributor (bits)
  __shared__ float4 s_grad[kWaves][kWave];   // upstream gradient rgb
  __shared__ float4 s_state[kWaves][kWave];  // T and the accumulated rgb before the next chunk
  __shared__ StagedSplat s_sp[kWaves][kWave];
  __shared__ uint32_t s_rel[kWaves][kWave];
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint32_t tile = tile_order[blockIdx.x];
  if (tile >= num_tiles) return;  // not reachable with a permutation; keeps reads in bounds
  load_exp_table(s_exp2);
  const uint32_t tx0 = (tile % tiles_x) * kTile, ty0 = (tile / tiles_x) * kTile;
  const uint32_t start = min(ranges[2 * tile], num_pairs);
  const uint32_t end = max(start, min(ranges[2 * tile + 1], num_pairs));
  const float tcx = float(tx0) + 8.0f, tcy = float(ty0) + 8.0f;  // the tile's centre, origin of the moments
  {
    // lane l sets up pixel l of the wave's block
    const uint32_t px = tx0 + lane_px(w, lane), py = ty0 + lane_py(w, lane);
    uint32_t last = 0;
    float4 c = make_float4(0.0f, 0.0f, 0.0f, 0.0f), g = c;
    if (px < width && py < height) {
      const size_t p = size_t(py) * width + px;
      last = min(last_contrib[p], end - start);
      c = out_rgba[p];
      g = v_out[p];
    }
    s_pix[w][lane] = make_float4(c.x, c.y, c.z, __uint_as_float(last));
    s_grad[w][lane] = make_float4(g.x, g.y, g.z, 0.0f);
    s_state[w][lane] = make_float4(1.0f, 0.0f, 0.0f, 0.0f);
  }
  __syncthreads();  // the exponential table; the rest is wave-private from here on
  uint32_t wave_last = __float_as_uint(s_pix[w][lane].w);
  const float4 gl = s_grad[w][lane];
  const bool g_finite = __builtin_isfinite(gl.x) && __builtin_isfinite(gl.y) && __builtin_isfinite(gl.z);
  const bool wave_g_finite = __builtin_amdgcn_readfirstlane(uint32_t(__ballot(!g_finite) == 0)) != 0;
  for (uint32_t off = 32; off > 0; off >>= 1) wave_last = max(wave_last, uint32_t(__shfl_xor(int(wave_last), off)));
  const uint32_t limit = min(__builtin_amdgcn_readfirstlane(wave_last), end - start);

  auto chunks = [&](auto guard) {
  constexpr bool kGuard = decltype(guard)::value;
  for (uint32_t rel0 = 0; rel0 < limit; rel0 += kWave) {
    // this chunk's candidates, culled against the wave's block and compacted in list order
    const uint32_t rel = rel0 + lane;
    StagedSplat cand;
    bool keep = false;
    if (rel < limit) {
      cand = stage_splat(splats, vals[start + rel], n);
      keep = kSkip ? ((reach_mask(cand, float(tx0) + 0.5f, float(ty0) + 0.5f) >> w) & 1u) != 0 : true;
    }
    const uint64_t kept = __ballot(keep);
    const uint32_t m = uint32_t(__popcll(kept));
    if (m == 0) continue;
    if (keep) {
      const uint32_t slot = uint32_t(__popcll(kept & ((uint64_t(1) << lane) - 1)));
      s_sp[w][slot] = cand;
      s_rel[w][slot] = rel;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    const bool mine = lane < m;
    const StagedSplat s = s_sp[w][mine ? lane : 0];
    const uint32_t srel = s_rel[w][mine ? lane : 0];
    float acc[kGrads];
#pragma unroll
    for (uint32_t q = 0; q < kGrads; ++q) acc[q] = 0.0f;
    float oT = 1.0f, oar = 0.0f, oag = 0.0f, oab = 0.0f;  // this lane's outgoing state of the previous step
    for (uint32_t t = 0; t < kWave + m - 1; ++t) {
      const int pi = int(t) - int(lane);
      const bool act = mine && pi >= 0 && pi < int(kWave);
      const uint32_t p = uint32_t(min(max(pi, 0), int(kWave) - 1));
      // incoming state: the previous lane's outgoing one; lane 0 reads the pixel's state from LDS
      float T = dpp_mov<kWaveShr1>(oT), ar = dpp_mov<kWaveShr1>(oar), ag = dpp_mov<kWaveShr1>(oag),
            ab = dpp_mov<kWaveShr1>(oab);
      if (lane == 0) {
        const float4 st = s_state[w][p];
        T = st.x, ar = st.y, ag = st.z, ab = st.w;
      }
      const float4 pc = s_pix[w][p];
      const float4 pg = s_grad[w][p];
      const float cx = float(tx0 + lane_px(w, p)) + 0.5f, cy = float(ty0 + lane_py(w, p)) + 0.5f;
      Eval e;  // evaluated in every lane, so that dx and dy are set where the terms below multiply them by 0
      const bool pass = evaluate<false>(s, cx, cy, e, s_exp2);
      const bool contrib = act && pass && srel < __float_as_uint(pc.w);
      const float alpha = contrib ? e.alpha : 0.0f;
      const float one_m = 1.0f - alpha;
      const float wgt = alpha * T;
      float d5 = wgt * pg.x, d6 = wgt * pg.y, d7 = wgt * pg.z;
      if constexpr (kGuard) {
        d5 = contrib ? d5 : 0.0f;
        d6 = contrib ? d6 : 0.0f;
        d7 = contrib ? d7 : 0.0f;
      }
      const float mr = s.r * wgt, mg = s.g * wgt, mb = s.bl * wgt;
      // as in the per-pixel kernel: after = (C_final - acc) - mine per channel
      const float g_rgb = __fmaf_rn(pg.z, s.bl, __fmaf_rn(pg.y, s.g, pg.x * s.r));
      const float g_after =
          __fmaf_rn(pg.z, (pc.z - ab) - mb, __fmaf_rn(pg.y, (pc.y - ag) - mg, pg.x * ((pc.x - ar) - mr)));
      const float dl_da = __fmaf_rn(T, g_rgb, -g_after * __builtin_amdgcn_rcpf(one_m));
      const float v = (contrib && e.oG < kAlphaMax) ? dl_da * e.G : 0.0f;
      // the per-pixel kernel's moments (pixel centre relative to the tile centre, exact), so that a sum of one
      // term gives that kernel's bits
      const float mu = cx - tcx, mt = cy - tcy;
      acc[0] += v;
      acc[1] += v * mu;
      acc[2] += v * mt;
      acc[3] += v * (mu * mu);
      acc[4] += v * (mu * mt);
      acc[5] += v * (mt * mt);
      acc[6] += d5;
      acc[7] += d6;
      acc[8] += d7;
      oT = T * one_m;
      oar = ar + mr;
      oag = ag + mg;
      oab = ab + mb;
      if (act && lane == m - 1) s_state[w][p] = make_float4(oT, oar, oag, oab);
    }
    // the splat's factors, as at the per-pixel kernel's flush, then its nine totals
    if (mine && s.idx != 0xFFFFFFFFu) {
      moments_to_grads(acc, s, tcx, tcy);
#pragma unroll
      for (uint32_t q = 0; q < kGrads; ++q) {
        if (acc[q] == 0.0f) continue;
        if constexpr (kDet)
          add_fixed(fixed, s.idx, q, acc[q]);
        else
          atomicAdd(splats_grad + size_t(s.idx) * kGrads + q, acc[q]);
      }
    }
    // the next chunk overwrites s_sp / s_rel, which this chunk's lanes read at its start only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
  };
  if (wave_g_finite)
    chunks(std::false_type{});
  else
    chunks(std::true_type{});
}

template <bool kSkip, bool kDet>
__global__ __launch_bounds__(kTilePixels) void k_backward_splat(GSR_BACKWARD_PARAMS) {
  backward_splat_tile<kSkip, kDet>(GSR_BACKWARD_ARGS);
}

// One block per 16x16 tile; the deterministic form under a name of its own, so that profiles keep the two apart.
template <bool kSkip>
__global__ __launch_bounds__(kTilePixels) __attribute__((amdgpu_waves_per_eu(6))) void k_backward(GSR_BACKWARD_PARAMS) {
  backward_tile<kSkip, false>(GSR_BACKWARD_ARGS);
}

template <bool kSkip>
__global__ __launch_bounds__(kTilePixels) void k_backward_det(GSR_BACKWARD_PARAMS) {
  backward_tile<kSkip, true>(GSR_BACKWARD_ARGS);
}

}  // namespace
}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_render_backward(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n,
                                          const gsr_bins* bins, uint32_t width, uint32_t height,
                                          const float* out_rgba, const float* final_T,
                                          const uint32_t* last_contrib, const float* v_out, float* splats_grad) {
  if (!ctx || !bins) return GSR_EINVAL;
  if (width == 0 || height == 0) return fail(ctx, GSR_EINVAL, "gsr_render_backward: empty image");
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  if (bins->tiles_x != tiles_x || bins->tiles_y != tiles_y)
    return fail(ctx, GSR_EINVAL, "gsr_render_backward: bins are for %ux%u tiles, image needs %ux%u", bins->tiles_x,
                bins->tiles_y, tiles_x, tiles_y);
  if (uint64_t(n) * kGrads >= (uint64_t(1) << 32))
    return fail(ctx, GSR_EOVERFLOW, "gsr_render_backward: n * 9 >= 2^32");
  if (!bins->ranges || (bins->num_pairs && !bins->vals) || (n && (!splats || !splats_grad)) || !out_rgba ||
      !final_T || !last_contrib || !v_out)
    return fail(ctx, GSR_EINVAL, "gsr_render_backward: null pointer");
  if (reinterpret_cast<uintptr_t>(out_rgba) % 16 || reinterpret_cast<uintptr_t>(v_out) % 16)
    return fail(ctx, GSR_EINVAL, "gsr_render_backward: out_rgba and v_out must be 16-byte aligned");
  const uint64_t num_tiles = uint64_t(tiles_x) * tiles_y;
  if (num_tiles >= (uint64_t(1) << 31)) return fail(ctx, GSR_EINVAL, "gsr_render_backward: too many tiles");
  gsr_status st = enter(ctx);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint64_t count = uint64_t(n) * kGrads;
  const bool det = ctx->deterministic && count;
  FixedSums fixed{nullptr, nullptr};
  const dim3 value_grid(uint32_t((count + kTilePixels - 1) / kTilePixels));
  if (det) {
    if ((st = grow(ctx, ctx->arena.grad_fixed, size_t(count) * 16 + size_t(n) * 4))) return st;
    fixed.words = static_cast<unsigned long long*>(ctx->arena.grad_fixed.ptr);
    fixed.flags = reinterpret_cast<uint32_t*>(fixed.words + 2 * count);
    hipLaunchKernelGGL(k_fixed_clear, value_grid, dim3(kTilePixels), 0, s, fixed, count, n);
  } else if (count) {
    hipLaunchKernelGGL(k_zero, dim3(uint32_t((count + 4 * kTilePixels - 1) / (4 * kTilePixels))), dim3(kTilePixels),
                       0, s, splats_grad, count, reinterpret_cast<uintptr_t>(splats_grad) % 16 == 0);
  }
  const uint32_t* order = raster_tile_order(ctx, s, bins, true, &st);
  if (!order) return st;
  auto kernel = ctx->raster_skip ? (det ? k_backward_det<true> : k_backward<true>)
                                 : (det ? k_backward_det<false> : k_backward<false>);
  if (ctx->backward_scheme == GSR_BACKWARD_PER_SPLAT)
    kernel = ctx->raster_skip ? (det ? k_backward_splat<true, true> : k_backward_splat<true, false>)
                              : (det ? k_backward_splat<false, true> : k_backward_splat<false, false>);
  timing_mark(ctx, GSR_STAGE_BACKWARD, s, false);
  hipLaunchKernelGGL(kernel, dim3(uint32_t(num_tiles)), dim3(kTilePixels), 0, s, splats, n, bins->vals,
                     bins->ranges, bins->num_pairs, tiles_x, width, height,
                     reinterpret_cast<const float4*>(out_rgba), last_contrib, reinterpret_cast<const float4*>(v_out),
                     splats_grad, fixed, order, uint32_t(num_tiles));
  timing_mark(ctx, GSR_STAGE_BACKWARD, s, true);
  if (det) hipLaunchKernelGGL(k_fixed_to_float, value_grid, dim3(kTilePixels), 0, s, fixed, splats_grad, count);
  return check_launch(ctx, "gsr_render_backward");
}
