// Forward rasterization: one 256-thread workgroup (four wave64, one 8x8 pixel block each) per 16x16 tile, one
// pixel per thread.
//
// The tile's depth-sorted splats are staged through LDS in batches of 256 (one record per thread), read back by
// every lane of a wave at the same address (LDS broadcast). While staging, each thread also marks which wave blocks
// its splat can reach; each wave then walks only those slots, in order, with a scalar loop over ballot bits. Each
// lane composites front to back in registers and stops when its pixel does; a wave leaves when all 64 lanes have;
// the workgroup stops staging batches once all 256 pixels are done (a counted barrier). [rasterize forward + adam kernel audit page, section 1 rows (a)
// and (b): batches of 256 staged records, a done counter for the tile, the per-lane !done loop exit]
#include "gsr_internal.hpp"
#include "raster_common.hpp"

namespace gsr {
namespace {

// kCull: each wave walks only the staged splats that can reach alpha >= 1/255 in its 8x8 block (reach_mask); the
// others are certain rejects for every lane of the wave, so skipping them changes no result.
// kExact: exp(-sigma) correctly rounded (fp64 series), so T and every stop decision are those of a plain fp32
// evaluation; otherwise the hardware exponential with the exact value only near the 1/255 threshold (evaluate's
// fast form without the clamp band): reject decisions are still exact, alpha and T carry the fast value's error
// (below 1e-6 relative per splat), so a pixel whose exact T' lies that close to 1e-4 may stop one splat apart.
template <bool kCull, bool kExact>
__global__ __launch_bounds__(kTilePixels) void k_forward(const float* __restrict__ splats, uint32_t n,
                                                         const uint32_t* __restrict__ vals,
                                                         const uint32_t* __restrict__ ranges, uint32_t num_pairs,
                                                         uint32_t tiles_x, uint32_t width, uint32_t height,
                                                         float4* __restrict__ out_rgba, float* __restrict__ final_T,
                                                         uint32_t* __restrict__ last_contrib,
                                                         const uint32_t* __restrict__ tile_order, uint32_t num_tiles,
                                                         uint32_t* __restrict__ tile_cost) {
  constexpr uint32_t kWaves = kTilePixels / kWave;
  __shared__ StagedSplat s_sp[kTilePixels];
  __shared__ double s_exp2[kExact ? 2 * kExpTabN : 64];  // the exponential's table (exp_neg_rn's or exp_rn's)
  __shared__ uint64_t s_mask[kWaves][kWaves];  // [reading wave][staging wave]: slots that can reach the reader
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint32_t tile = tile_order[blockIdx.x];  // slowest expected first (a permutation of the tiles)
  if (tile >= num_tiles) return;                 // not reachable with a permutation; keeps reads in bounds
  if constexpr (kExact)
    load_exp_neg_table(s_exp2);  // the first batch barrier orders it
  else
    load_exp_table(s_exp2);
  const uint32_t tx0 = (tile % tiles_x) * kTile, ty0 = (tile / tiles_x) * kTile;
  const uint32_t px = tx0 + lane_px(w, lane), py = ty0 + lane_py(w, lane);
  const bool inside = px < width && py < height;
  const uint32_t start = min(ranges[2 * tile], num_pairs);
  const uint32_t end = max(start, min(ranges[2 * tile + 1], num_pairs));
  const float cx = float(px) + 0.5f, cy = float(py) + 0.5f;

  float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
  uint32_t last = 0, last_stop = 0;
  uint32_t walked = 0;  // splats this wave evaluated (wave-uniform): the tile's cost for the launch order
  // A lane whose pixel has stopped (or lies outside the image) moves its centre to +inf: sigma is then inf or NaN
  // for every later splat, which evaluate() rejects, so finished lanes need no test of their own.
  const float kFar = __builtin_huge_valf();
  float cxe = inside ? cx : kFar;
  for (uint32_t b0 = start; b0 < end; b0 += kTilePixels) {
    if (__syncthreads_count(cxe == kFar) == int(kTilePixels)) break;  // also orders the previous batch's reads
    const uint32_t k = b0 + tid;
    uint32_t reach = 0;
    if (k < end) {
      const StagedSplat st = stage_splat(splats, vals[k], n);
      s_sp[tid] = st;
      reach = kCull ? reach_mask(st, float(tx0) + 0.5f, float(ty0) + 0.5f) : 0xFu;
    }
#pragma unroll
    for (uint32_t q = 0; q < kWaves; ++q) {
      const uint64_t bits = __ballot((reach >> q) & 1u);
      if (lane == 0) s_mask[q][w] = bits;
    }
    __syncthreads();
    if (__ballot(cxe != kFar) == 0) continue;  // this wave is finished; keep joining the barriers
    const uint32_t pos0 = b0 - start + 1;
    for (uint32_t sw = 0; sw < kWaves; ++sw) {
      uint64_t m = uniform64(s_mask[w][sw]);
      while (m) {
        const uint32_t j = sw * kWave + uint32_t(__builtin_ctzll(m));
        m &= m - 1;
        // the whole record in three 16-byte reads from one address register (the loop reads every field of it
        // in some branch; read lazily each branch would need its own address)
        const float4* rec = reinterpret_cast<const float4*>(&s_sp[j]);
        const float4 q0 = rec[0], q1 = rec[1], q2 = rec[2];
        StagedSplat s;
        s.x = q0.x, s.y = q0.y, s.ha = q0.z, s.b = q0.w;
        s.hc = q1.x, s.o = q1.y, s.r = q1.z, s.g = q1.w;
        s.bl = q2.x, s.lr = q2.y, s.hb = q2.z, s.idx = __float_as_uint(q2.w);
        // o is read in this load, not in a fourth one inside the branches (which needs its own address register)
        asm volatile("" ::"v"(s.o));
        ++walked;
        Eval e;
        if (evaluate<kExact, kExact>(s, cxe, cy, e, s_exp2)) {
          float alpha = e.alpha;
          float next_T = T * (1.0f - alpha);
          // A pixel that would fall below the stop threshold here does not composite this splat and stops. Rare
          // (once per pixel), so behind a wave test: such a lane keeps its last contributor aside and takes
          // alpha = 0, which makes the update below leave T and its colours as they are (r 0 = +-0 added to a sum
          // that starts at +0 and never becomes -0; binned colours are finite), and its centre moves to +inf.
          if (__builtin_amdgcn_ballot_w64(next_T < kTStop) != 0) {
            const bool stop = next_T < kTStop;
            last_stop = stop ? last : last_stop;
            alpha = stop ? 0.0f : alpha;
            next_T = stop ? T : next_T;
            cxe = stop ? kFar : cxe;
          }
          // The colour sums use a fused multiply-add (one rounding per splat instead of two): the image stays
          // within 2e-7 of the two-rounding sum, far inside its bar, and no decision depends on it (T and the
          // stop test keep their plain fp32 operations).
          const float wgt = alpha * T;
          cr = __fmaf_rn(s.r, wgt, cr);
          cg = __fmaf_rn(s.g, wgt, cg);
          cb = __fmaf_rn(s.bl, wgt, cb);
          T = next_T;
          last = pos0 + j;
        }
        if (__ballot(cxe != kFar) == 0) {
          sw = kWaves;
          break;
        }
      }
    }
  }
  // a stopped pixel's last contributor is the one kept aside (the update at its stopping splat overwrote it)
  if (inside && cxe == kFar) last = last_stop;
  if (inside) {
    const size_t p = size_t(py) * width + px;
    out_rgba[p] = make_float4(cr, cg, cb, 1.0f - T);
    final_T[p] = T;
    last_contrib[p] = last;
  }
  if (lane == 0) tile_cost[4 * size_t(tile) + w] = walked;
}

// Scratch of gsr_render_forward_noalloc, one copy per device (it lives as long as the library is loaded):
// [0, kNoAllocMaxTiles) the tiles' launch order, [kNoAllocMaxTiles, 5 kNoAllocMaxTiles) the four per-wave walk
// counts of each tile from the last no-alloc forward on the device, which rank the next one's launch order. Host code
// uses the address noalloc_setup looks up, never the array's name (which is a host-side stand-in).
constexpr uint32_t kNoAllocMaxTiles = 65536;
__device__ __align__(256) uint32_t scratch[5 * kNoAllocMaxTiles];

using ForwardKernel = void (*)(const float*, uint32_t, const uint32_t*, const uint32_t*, uint32_t, uint32_t, uint32_t,
                               uint32_t, float4*, float*, uint32_t*, const uint32_t*, uint32_t, uint32_t*);

// The forward kernel the context's options select (GSR_OPT_RASTER_SKIP, GSR_OPT_FORWARD_EXP).
ForwardKernel forward_kernel(const gsr_ctx* ctx) {
  const bool exact = ctx->forward_exp == GSR_EXP_EXACT;
  if (ctx->raster_skip) return exact ? k_forward<true, true> : k_forward<true, false>;
  return exact ? k_forward<false, true> : k_forward<false, false>;
}

}  // namespace

gsr_status noalloc_setup(gsr_ctx* ctx) {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return hip_fail(ctx, e != hipSuccess ? e : hipErrorInvalidSymbol, "noalloc scratch");
  ctx->noalloc_scratch = static_cast<uint32_t*>(p);
  return GSR_OK;
}

}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_render_forward(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n,
                                         const gsr_bins* bins, uint32_t width, uint32_t height, float* out_rgba,
                                         float* final_T, uint32_t* last_contrib) {
  if (!ctx || !bins) return GSR_EINVAL;
  if (width == 0 || height == 0) return fail(ctx, GSR_EINVAL, "gsr_render_forward: empty image");
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  if (bins->tiles_x != tiles_x || bins->tiles_y != tiles_y)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward: bins are for %ux%u tiles, image needs %ux%u", bins->tiles_x,
                bins->tiles_y, tiles_x, tiles_y);
  if (!bins->ranges || (bins->num_pairs && !bins->vals) || (n && !splats) || !out_rgba || !final_T || !last_contrib)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward: null pointer");
  if (reinterpret_cast<uintptr_t>(out_rgba) % 16)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward: out_rgba must be 16-byte aligned");
  const uint64_t num_tiles = uint64_t(tiles_x) * tiles_y;
  if (num_tiles >= (uint64_t(1) << 31)) return fail(ctx, GSR_EINVAL, "gsr_render_forward: too many tiles");
  gsr_status st = enter(ctx);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t* order = raster_tile_order(ctx, s, bins, false, &st);
  if (!order) return st;
  // the walk lengths of this forward rank the tiles of the next raster launch on this grid
  if ((st = grow(ctx, ctx->arena.tile_cost, size_t(num_tiles) * 16))) return st;
  timing_mark(ctx, GSR_STAGE_FORWARD, s, false);
  hipLaunchKernelGGL(forward_kernel(ctx), dim3(uint32_t(num_tiles)), dim3(kTilePixels), 0, s, splats, n, bins->vals,
                     bins->ranges, bins->num_pairs, tiles_x, width, height, reinterpret_cast<float4*>(out_rgba),
                     final_T, last_contrib, order, uint32_t(num_tiles),
                     static_cast<uint32_t*>(ctx->arena.tile_cost.ptr));
  timing_mark(ctx, GSR_STAGE_FORWARD, s, true);
  if ((st = check_launch(ctx, "gsr_render_forward"))) return st;
  ctx->cost_tiles = num_tiles;
  return GSR_OK;
}

extern "C" gsr_status gsr_render_forward_noalloc(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n,
                                                 const gsr_bins* bins, uint32_t width, uint32_t height,
                                                 float* out_rgba, float* final_T, uint32_t* last_contrib) {
  if (!ctx || !bins) return GSR_EINVAL;
  if (width == 0 || height == 0) return fail(ctx, GSR_EINVAL, "gsr_render_forward_noalloc: empty image");
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  const uint64_t num_tiles = uint64_t(tiles_x) * tiles_y;
  if (num_tiles > kNoAllocMaxTiles)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward_noalloc: %llu tiles exceed the scratch's %u (use "
                "gsr_render_forward)", (unsigned long long)num_tiles, kNoAllocMaxTiles);
  if (bins->tiles_x != tiles_x || bins->tiles_y != tiles_y)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward_noalloc: bins are for %ux%u tiles, image needs %ux%u",
                bins->tiles_x, bins->tiles_y, tiles_x, tiles_y);
  if (!bins->ranges || (bins->num_pairs && !bins->vals) || (n && !splats) || !out_rgba || !final_T || !last_contrib)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward_noalloc: null pointer");
  if (reinterpret_cast<uintptr_t>(out_rgba) % 16)
    return fail(ctx, GSR_EINVAL, "gsr_render_forward_noalloc: out_rgba must be 16-byte aligned");
  if (!ctx->noalloc_scratch) return fail(ctx, GSR_EHIP, "gsr_render_forward_noalloc: no scratch on this device");
  gsr_status st = enter(ctx);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* order = ctx->noalloc_scratch;
  uint32_t* cost = ctx->noalloc_scratch + kNoAllocMaxTiles;
  // Rank by the walk counts the previous no-alloc forward on this device left (a valid permutation whatever they
  // hold; the order changes no result), then render; this forward leaves its own counts for the next one.
  launch_tile_order(s, bins->ranges, ctx->tile_order == GSR_ORDER_COST ? cost : nullptr, uint32_t(num_tiles),
                    bins->num_pairs, order, ctx->tile_order == GSR_ORDER_NONE);
  timing_mark(ctx, GSR_STAGE_FORWARD, s, false);
  hipLaunchKernelGGL(forward_kernel(ctx), dim3(uint32_t(num_tiles)), dim3(kTilePixels), 0, s, splats, n, bins->vals,
                     bins->ranges, bins->num_pairs, tiles_x, width, height, reinterpret_cast<float4*>(out_rgba),
                     final_T, last_contrib, static_cast<const uint32_t*>(order), uint32_t(num_tiles), cost);
  timing_mark(ctx, GSR_STAGE_FORWARD, s, true);
  return check_launch(ctx, "gsr_render_forward_noalloc");
}
